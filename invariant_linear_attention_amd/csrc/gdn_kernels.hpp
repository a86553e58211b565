// gdn_kernels.hpp -- gfx950 kernels of the batch-invariant gated delta rule forward.
//
// The recurrence (gated delta rule, Yang/Kautz/Hatamizadeh, ICLR 2025), per sequence
// and value head, token by token:
//     a_t = exp(g_t),  S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t
// run as one recurrent walk for prefill and for decode, each sequence against its own
// state only (page "Defending Against the Training-Inference Numeric Mismatch in RL
// (Especially Linear Attention)", section 3.2).
//
// How one state row j (dk fp32 values, row j of the dv x dk matrix S) is computed.
// This fixes every bit of the result; nothing below depends on the batch, on where a
// sequence sits in it, on the launch shape or on the kernel (prefill or decode):
//
//   * The row lives in the registers of one lane quad.  Lane l (0..3) holds the
//     columns 16c + 4l + e for chunk c = 0 .. dk/16 - 1 and e = 0..3.
//   * A dot product of the row with a dk-vector x is a fixed tree: each lane forms
//     "leaf" sums over 8 columns (4 when dk = 16) -- two consecutive chunks, columns in
//     (c, e) order, as one multiply followed by fused multiply-adds -- then adds its
//     leaves pairwise ((L0+L1)+(L2+L3)), then the quad adds across lanes l^1 and
//     then l^2 with DPP.  Every lane of the quad ends with the same bits.
//   * Per token, with ptil = S_{t-1} . k_t (that tree):
//         a = 2^(g * log2 e) (hardware exp2),  p = a * ptil,  u = beta * (v_j - p)
//         S[i] = fma(a, S[i], u * k_t[i])        for every column i
//         o_j  = S_t . q_t                       (the same tree)
//     and in prefill the next token's ptil = S_t . k_{t+1} is formed in the same sweep,
//     with the same tree, which is the value a fresh sweep would give.
//
// Rows never interact, so how rows are spread over quads, waves and workgroups is free
// (a launch-shape choice); within a row the arithmetic above is fixed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.hpp"

#pragma clang fp contract(off)

namespace gdn {

// ----------------------------------------------------------------- numerics

// exp(g) as 2^(g log2 e) with the hardware base-2 exponential.
__device__ __forceinline__ float decay_factor(float g) {
    return __builtin_amdgcn_exp2f(g * 1.44269504088896340736f);
}

// u_j = beta * (v_j - a * ptil_j): the delta-rule write coefficient.
__device__ __forceinline__ float delta_coeff(float a, float ptil, float v, float beta) {
    const float p = a * ptil;
    return beta * (v - p);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t x = __float_as_uint(f);
    if ((x & 0x7fffffffu) > 0x7f800000u) return (x >> 16) | 0x0040u;
    x += 0x7fffu + ((x >> 16) & 1u);
    return x >> 16;
}

// Sum over the four lanes of a quad: partner l^1 (quad_perm 1,0,3,2), then l^2
// (quad_perm 2,3,0,1).  Addition is commutative, so all four lanes get equal bits.
__device__ __forceinline__ float quad_sum(float x) {
    x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
    x = x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
    return x;
}

template <int DK>
struct Geo {
    static_assert(DK == 16 || DK == 32 || DK == 64 || DK == 128, "unsupported dk");
    static constexpr int C = DK / 4;             // columns per lane
    static constexpr int NCH = C / 4;            // 4-column chunks per lane
    static constexpr int LF = (C < 8) ? C : 8;   // leaf length (columns)
    static constexpr int CPL = LF / 4;           // chunks per leaf
    static constexpr int NLEAF = C / LF;         // leaves per lane
};

template <int N>
__device__ __forceinline__ float leaf_tree(const float (&x)[N]) {
    if constexpr (N == 1) {
        return x[0];
    } else if constexpr (N == 2) {
        return x[0] + x[1];
    } else {
        static_assert(N == 4, "leaf count");
        return (x[0] + x[1]) + (x[2] + x[3]);
    }
}

// res[r] = S[r] . x  for the R rows held by this lane (all quad lanes get the result).
template <int DK, int R>
__device__ __forceinline__ void row_dots(const float (&S)[R][DK / 4], const float (&x)[DK / 4], float (&res)[R]) {
    using G = Geo<DK>;
    float acc[R][G::NLEAF];
#pragma unroll
    for (int c = 0; c < G::NCH; ++c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * c + e;
            const int lf = c / G::CPL;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if ((c % G::CPL) == 0 && e == 0)
                    acc[r][lf] = S[r][i] * x[i];
                else
                    acc[r][lf] = __builtin_fmaf(S[r][i], x[i], acc[r][lf]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) res[r] = quad_sum(leaf_tree<G::NLEAF>(acc[r]));
}

// One token's state update and read-out for the R rows of this lane:
//   S[r][i] = fma(a, S[r][i], u[r] * kc[i]);  o[r] = S[r] . q
// and, when NEXT, ptil[r] = S[r] . kn with kn (the next token's key) copied into
// registers on the way.  qchunk(c) / kchunk(c) return 4 columns of chunk c.
template <int DK, int R, bool NEXT, class QF, class KF>
__device__ __forceinline__ void update_sweep(float (&S)[R][DK / 4], const float (&kc)[DK / 4], float (&kn)[DK / 4],
                                             QF qchunk, KF kchunk, float a, const float (&u)[R], float (&o)[R],
                                             float (&ptil)[R]) {
    using G = Geo<DK>;
    float ao[R][G::NLEAF];
    float ap[R][G::NLEAF];
#pragma unroll
    for (int c = 0; c < G::NCH; ++c) {
        const float4 q4 = qchunk(c);
        const float qe[4] = {q4.x, q4.y, q4.z, q4.w};
        float ke[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NEXT) {
            const float4 k4 = kchunk(c);
            ke[0] = k4.x; ke[1] = k4.y; ke[2] = k4.z; ke[3] = k4.w;
            kn[4 * c + 0] = k4.x; kn[4 * c + 1] = k4.y; kn[4 * c + 2] = k4.z; kn[4 * c + 3] = k4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * c + e;
            const int lf = c / G::CPL;
            const bool first = (c % G::CPL) == 0 && e == 0;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float w = u[r] * kc[i];
                const float s = __builtin_fmaf(a, S[r][i], w);
                S[r][i] = s;
                if (first) {
                    ao[r][lf] = s * qe[e];
                    if constexpr (NEXT) ap[r][lf] = s * ke[e];
                } else {
                    ao[r][lf] = __builtin_fmaf(s, qe[e], ao[r][lf]);
                    if constexpr (NEXT) ap[r][lf] = __builtin_fmaf(s, ke[e], ap[r][lf]);
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        o[r] = quad_sum(leaf_tree<G::NLEAF>(ao[r]));
        if constexpr (NEXT) ptil[r] = quad_sum(leaf_tree<G::NLEAF>(ap[r]));
    }
}

// ------------------------------------------------------------------ io types

struct IoBf16 {
    static constexpr int VEC = 8;  // elements per 16-byte vector
    static constexpr int ID = GDN_BF16;
    __device__ static void unpack(const uint4 &raw, float *f) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i + 0] = bf16_to_f32(w[i] & 0xffffu);
            f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
        }
    }
    // Four consecutive elements starting at element index idx (8-byte aligned).
    __device__ static float4 load4(const void *base, size_t idx) {
        const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
        return make_float4(bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xffffu),
                           bf16_to_f32(w.y >> 16));
    }
    __device__ static float load1(const void *base, size_t idx) {
        return bf16_to_f32(static_cast<const uint16_t *>(base)[idx]);
    }
    __device__ static void store1(void *base, size_t idx, float f) {
        static_cast<uint16_t *>(base)[idx] = static_cast<uint16_t>(f32_to_bf16_rne(f));
    }
};

struct IoF32 {
    static constexpr int VEC = 4;
    static constexpr int ID = GDN_F32;
    __device__ static void unpack(const uint4 &raw, float *f) {
        f[0] = __uint_as_float(raw.x);
        f[1] = __uint_as_float(raw.y);
        f[2] = __uint_as_float(raw.z);
        f[3] = __uint_as_float(raw.w);
    }
    __device__ static float4 load4(const void *base, size_t idx) {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
    }
    __device__ static float load1(const void *base, size_t idx) { return static_cast<const float *>(base)[idx]; }
    __device__ static void store1(void *base, size_t idx, float f) { static_cast<float *>(base)[idx] = f; }
};

// ------------------------------------------------------------- prefill kernel

// Tokens staged per block through LDS (double-buffered).
constexpr int kTokenBlock = 16;

template <int DK, class IO, int R, int NW>
struct PrefillShape {
    static constexpr int TB = kTokenBlock;
    static constexpr int RW = NW * 16 * R;          // rows per workgroup
    static constexpr int NT = NW * 64;              // threads per workgroup
    static constexpr int KVEC = DK / IO::VEC;       // 16-byte vectors per key/query row
    static constexpr int VVEC = RW / IO::VEC;       // 16-byte vectors per value row slice
    static constexpr int KITEMS = (TB + 1) * KVEC;  // keys: TB tokens + the next block's first
    static constexpr int QITEMS = TB * KVEC;
    static constexpr int VITEMS = TB * VVEC;
    static constexpr int KSLOTS = (KITEMS + NT - 1) / NT;
    static constexpr int QSLOTS = (QITEMS + NT - 1) / NT;
    static constexpr int VSLOTS = (VITEMS + NT - 1) / NT;
    static_assert(2 * TB <= NT, "gate/beta staging needs 2*TB threads");
    static_assert(RW % IO::VEC == 0, "row slice must be whole vectors");
};

template <int DK, class IO, int R, int NW>
struct PrefillLds {
    using Sh = PrefillShape<DK, IO, R, NW>;
    float k[2][Sh::TB + 1][DK];
    float q[2][Sh::TB][DK];
    float v[2][Sh::TB][Sh::RW];
    float a[2][Sh::TB];
    float b[2][Sh::TB];
};

// Global -> register stage of one token block (issued early), then register -> LDS.
template <int DK, class IO, int R, int NW>
struct Stager {
    using Sh = PrefillShape<DK, IO, R, NW>;
    uint4 kr[Sh::KSLOTS];
    uint4 qr[Sh::QSLOTS];
    uint4 vr[Sh::VSLOTS];
    float gb;

    __device__ __forceinline__ void load(const PrefillParams &p, int64_t t0, int64_t te, int kh, int h, int row0,
                                         int tid) {
        const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < Sh::KSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            const int ti = it / Sh::KVEC, vec = it % Sh::KVEC;
            const int64_t t = t0 + ti;
            kr[s] = zero;
            if (it < Sh::KITEMS && t < te)
                kr[s] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.k) +
                                                         ((size_t)(t * p.hk + kh) * DK + (size_t)vec * IO::VEC) *
                                                             (IO::VEC == 8 ? 2 : 4));
        }
#pragma unroll
        for (int s = 0; s < Sh::QSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            const int ti = it / Sh::KVEC, vec = it % Sh::KVEC;
            const int64_t t = t0 + ti;
            qr[s] = zero;
            if (it < Sh::QITEMS && t < te)
                qr[s] = *reinterpret_cast<const uint4 *>(static_cast<const char *>(p.q) +
                                                         ((size_t)(t * p.hk + kh) * DK + (size_t)vec * IO::VEC) *
                                                             (IO::VEC == 8 ? 2 : 4));
        }
#pragma unroll
        for (int s = 0; s < Sh::VSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            const int ti = it / Sh::VVEC, vec = it % Sh::VVEC;
            const int64_t t = t0 + ti;
            vr[s] = zero;
            if (it < Sh::VITEMS && t < te)
                vr[s] = *reinterpret_cast<const uint4 *>(
                    static_cast<const char *>(p.v) +
                    ((size_t)(t * p.hv + h) * p.dv + row0 + (size_t)vec * IO::VEC) * (IO::VEC == 8 ? 2 : 4));
        }
        gb = 0.f;
        if (tid < 2 * Sh::TB) {
            const int ti = tid % Sh::TB;
            const int64_t t = t0 + ti;
            if (t < te) gb = (tid < Sh::TB) ? p.g[t * p.hv + h] : p.beta[t * p.hv + h];
        }
    }

    __device__ __forceinline__ void store(PrefillLds<DK, IO, R, NW> &L, int buf, int tid) const {
#pragma unroll
        for (int s = 0; s < Sh::KSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            if (it < Sh::KITEMS) {
                const int ti = it / Sh::KVEC, vec = it % Sh::KVEC;
                float f[IO::VEC];
                IO::unpack(kr[s], f);
#pragma unroll
                for (int x = 0; x < IO::VEC; x += 4)
                    *reinterpret_cast<float4 *>(&L.k[buf][ti][vec * IO::VEC + x]) =
                        make_float4(f[x], f[x + 1], f[x + 2], f[x + 3]);
            }
        }
#pragma unroll
        for (int s = 0; s < Sh::QSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            if (it < Sh::QITEMS) {
                const int ti = it / Sh::KVEC, vec = it % Sh::KVEC;
                float f[IO::VEC];
                IO::unpack(qr[s], f);
#pragma unroll
                for (int x = 0; x < IO::VEC; x += 4)
                    *reinterpret_cast<float4 *>(&L.q[buf][ti][vec * IO::VEC + x]) =
                        make_float4(f[x], f[x + 1], f[x + 2], f[x + 3]);
            }
        }
#pragma unroll
        for (int s = 0; s < Sh::VSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            if (it < Sh::VITEMS) {
                const int ti = it / Sh::VVEC, vec = it % Sh::VVEC;
                float f[IO::VEC];
                IO::unpack(vr[s], f);
#pragma unroll
                for (int x = 0; x < IO::VEC; x += 4)
                    *reinterpret_cast<float4 *>(&L.v[buf][ti][vec * IO::VEC + x]) =
                        make_float4(f[x], f[x + 1], f[x + 2], f[x + 3]);
            }
        }
        if (tid < Sh::TB)
            L.a[buf][tid] = decay_factor(gb);
        else if (tid < 2 * Sh::TB)
            L.b[buf][tid - Sh::TB] = gb;
    }
};

// One workgroup = (sequence n = blockIdx.z, value head h = blockIdx.y, row tile blockIdx.x).
template <int DK, class IO, int R, int NW>
__global__ __launch_bounds__(NW * 64) void gdn_prefill_kernel(PrefillParams p) {
    using Sh = PrefillShape<DK, IO, R, NW>;
    constexpr int C = DK / 4, NCH = C / 4, TB = Sh::TB;
    __shared__ PrefillLds<DK, IO, R, NW> L;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l = lane & 3, qd = lane >> 2;
    const int n = blockIdx.z, h = blockIdx.y;
    const int row0 = blockIdx.x * Sh::RW;
    const int kh = h / (p.hv / p.hk);

    // Sequence bounds, clamped into [0, T] so that a malformed cu_seqlens cannot
    // send the kernel outside the buffers.
    int64_t tb = p.cu_seqlens[n], te = p.cu_seqlens[n + 1];
    tb = tb < 0 ? 0 : (tb > p.total_tokens ? p.total_tokens : tb);
    te = te < tb ? tb : (te > p.total_tokens ? p.total_tokens : te);
    const int64_t len = te - tb;

    const int wrow = wave * 16 * R + qd;  // this lane's first row inside the tile (rows wrow + 16 r)
    const size_t state_row0 = ((size_t)n * p.hv + h) * p.dv + row0 + wrow;

    float S[R][C];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (p.h0) x = *reinterpret_cast<const float4 *>(p.h0 + (state_row0 + 16 * r) * DK + 16 * c + 4 * l);
            S[r][4 * c + 0] = x.x; S[r][4 * c + 1] = x.y; S[r][4 * c + 2] = x.z; S[r][4 * c + 3] = x.w;
        }
    }

    if (len > 0) {
        const int nblk = (int)((len + TB - 1) / TB);
        Stager<DK, IO, R, NW> st;
        st.load(p, tb, te, kh, h, row0, tid);
        st.store(L, 0, tid);
        __syncthreads();

        float kA[C], kB[C], ptil[R];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float4 x = *reinterpret_cast<const float4 *>(&L.k[0][0][16 * c + 4 * l]);
            kA[4 * c + 0] = x.x; kA[4 * c + 1] = x.y; kA[4 * c + 2] = x.z; kA[4 * c + 3] = x.w;
        }
        row_dots<DK, R>(S, kA, ptil);

        for (int blk = 0; blk < nblk; ++blk) {
            const int buf = blk & 1;
            const int64_t t0 = tb + (int64_t)blk * TB;
            if (blk + 1 < nblk) st.load(p, t0 + TB, te, kh, h, row0, tid);
            const int nt = (int)((te - t0) < TB ? (te - t0) : TB);

            auto step = [&](float (&kc)[C], float (&kn)[C], int ti) {
                const float a = L.a[buf][ti];
                const float beta = L.b[buf][ti];
                float u[R], o[R];
#pragma unroll
                for (int r = 0; r < R; ++r) u[r] = delta_coeff(a, ptil[r], L.v[buf][ti][wrow + 16 * r], beta);
                update_sweep<DK, R, true>(
                    S, kc, kn,
                    [&](int c) { return *reinterpret_cast<const float4 *>(&L.q[buf][ti][16 * c + 4 * l]); },
                    [&](int c) { return *reinterpret_cast<const float4 *>(&L.k[buf][ti + 1][16 * c + 4 * l]); }, a,
                    u, o, ptil);
                float ov = o[0];
#pragma unroll
                for (int r = 1; r < R; ++r)
                    if (l == r) ov = o[r];
                if (l < R) IO::store1(p.out, (size_t)((t0 + ti) * p.hv + h) * p.dv + row0 + wrow + 16 * l, ov);
            };

            int ti = 0;
            for (; ti + 1 < nt; ti += 2) {
                step(kA, kB, ti);
                step(kB, kA, ti + 1);
            }
            if (ti < nt) step(kA, kB, ti);

            if (blk + 1 < nblk) st.store(L, buf ^ 1, tid);
            __syncthreads();
        }
    }

    if (p.hT) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                *reinterpret_cast<float4 *>(p.hT + (state_row0 + 16 * r) * DK + 16 * c + 4 * l) =
                    make_float4(S[r][4 * c + 0], S[r][4 * c + 1], S[r][4 * c + 2], S[r][4 * c + 3]);
        }
    }
}

// -------------------------------------------------------------- decode kernel

// One workgroup = (batch row b = blockIdx.z, value head h = blockIdx.y, row tile blockIdx.x).
template <int DK, class IO, int R, int NW>
__global__ __launch_bounds__(NW * 64) void gdn_decode_kernel(DecodeParams p) {
    constexpr int C = DK / 4, NCH = C / 4;
    constexpr int RW = NW * 16 * R;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l = lane & 3, qd = lane >> 2;
    const int b = blockIdx.z, h = blockIdx.y;
    const int row0 = blockIdx.x * RW;
    const int kh = h / (p.hv / p.hk);
    const int wrow = wave * 16 * R + qd;
    const size_t orow = ((size_t)b * p.hv + h) * p.dv + row0 + wrow;

    const int slot = p.state_idx ? p.state_idx[b] : b;
    if (slot < 0 || slot >= p.pool_size) {  // padding row: zero output, no state access
        if (l < R) IO::store1(p.out, orow + 16 * l, 0.f);
        return;
    }
    float *st = p.pool + (((size_t)slot * p.hv + h) * p.dv + row0 + wrow) * DK;

    float S[R][C];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float4 x = *reinterpret_cast<const float4 *>(st + (size_t)16 * r * DK + 16 * c + 4 * l);
            S[r][4 * c + 0] = x.x; S[r][4 * c + 1] = x.y; S[r][4 * c + 2] = x.z; S[r][4 * c + 3] = x.w;
        }
    }
    float kx[C], qx[C];
    const size_t qk0 = ((size_t)b * p.hk + kh) * DK;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const float4 k4 = IO::load4(p.k, qk0 + 16 * c + 4 * l);
        const float4 q4 = IO::load4(p.q, qk0 + 16 * c + 4 * l);
        kx[4 * c + 0] = k4.x; kx[4 * c + 1] = k4.y; kx[4 * c + 2] = k4.z; kx[4 * c + 3] = k4.w;
        qx[4 * c + 0] = q4.x; qx[4 * c + 1] = q4.y; qx[4 * c + 2] = q4.z; qx[4 * c + 3] = q4.w;
    }
    const float a = decay_factor(p.g[(size_t)b * p.hv + h]);
    const float beta = p.beta[(size_t)b * p.hv + h];

    float ptil[R], u[R], o[R];
    row_dots<DK, R>(S, kx, ptil);
#pragma unroll
    for (int r = 0; r < R; ++r) u[r] = delta_coeff(a, ptil[r], IO::load1(p.v, orow + 16 * r), beta);
    float unused[C];
    update_sweep<DK, R, false>(
        S, kx, unused,
        [&](int c) { return make_float4(qx[4 * c + 0], qx[4 * c + 1], qx[4 * c + 2], qx[4 * c + 3]); },
        [&](int c) { return make_float4(0.f, 0.f, 0.f, 0.f); }, a, u, o, ptil);

#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            *reinterpret_cast<float4 *>(st + (size_t)16 * r * DK + 16 * c + 4 * l) =
                make_float4(S[r][4 * c + 0], S[r][4 * c + 1], S[r][4 * c + 2], S[r][4 * c + 3]);
    }
    float ov = o[0];
#pragma unroll
    for (int r = 1; r < R; ++r)
        if (l == r) ov = o[r];
    if (l < R) IO::store1(p.out, orow + 16 * l, ov);
}

// ------------------------------------------------------------ launch helpers

template <int DK, class IO, int R, int NW>
hipError_t launch_prefill_t(const PrefillParams &p, hipStream_t s) {
    constexpr int RW = NW * 16 * R;
    dim3 grid(p.dv / RW, p.hv, p.n_seqs), block(NW * 64);
    void *args[] = {const_cast<PrefillParams *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gdn_prefill_kernel<DK, IO, R, NW>), grid, block, args, 0,
                           s);
}

template <int DK, class IO, int R, int NW>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t s) {
    constexpr int RW = NW * 16 * R;
    dim3 grid(p.dv / RW, p.hv, p.batch), block(NW * 64);
    void *args[] = {const_cast<DecodeParams *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gdn_decode_kernel<DK, IO, R, NW>), grid, block, args, 0,
                           s);
}

}  // namespace gdn
