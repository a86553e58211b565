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
//   * Columns are grouped into "leaves" of 8 (4 when dk = 16).  With the column
//     index written as 16c + 4l + e (l, e in 0..3, c in 0..dk/16-1), leaf (l, s)
//     holds the columns with l fixed and c in {2s, 2s+1}, in (c, e) order (for
//     dk = 16: c = 0 only).  A leaf sum is one multiply followed by fused
//     multiply-adds in that order.
//   * A dot product of the row with a dk-vector is a fixed binary tree over the
//     leaves, in the leaf order m = l * (leaves per l) + s: pairs (2i, 2i+1) first,
//     then pairs of pairs, and so on.
//   * Per token, with ptil = S_{t-1} . k_t (that tree):
//         a = 2^(g * log2 e) (hardware exp2),  ab = a * beta,  bv = beta * v_j
//         u = fma(-ab, ptil, bv)                 (= beta (v_j - a ptil))
//         S[i] = fma(a, S[i], u * k_t[i])        for every column i
//         o_j  = S_t . q_t                       (the same tree)
//     and in prefill the next token's ptil = S_t . k_{t+1} is formed in the same
//     pass, which is the value a separate pass would give.
//
// How a row is spread over lanes is a launch choice that cannot change those bits:
// L lanes (4, 8 or 16, consecutive lanes of one DPP row) hold one row, each lane a
// contiguous run of leaves; the lanes first add their own leaves pairwise, then the
// remaining tree levels run across lanes with DPP (partners l^1 and l^2 inside a
// quad, then half-row and row mirrors), so every level adds the same two partial
// sums whichever lanes hold them.  Rows never interact, so the rows per lane, waves
// per workgroup and workgroups per head are free as well.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <stdint.h>

#include "gdn_internal.hpp"

#pragma clang fp contract(off)

namespace gdn {

// ----------------------------------------------------------------- numerics

// exp(g) as 2^(g log2 e) with the hardware base-2 exponential.
__device__ __forceinline__ float decay_factor(float g) {
    return __builtin_amdgcn_exp2f(g * 1.44269504088896340736f);
}

// The delta-rule write coefficient u_j = beta (v_j - a ptil_j), evaluated as
// fma(-ab, ptil_j, bv_j) with ab = a * beta (once per token and head) and
// bv_j = beta * v_j (once per token and row, when v is staged).
__device__ __forceinline__ float scaled_decay(float a, float beta) { return a * beta; }
__device__ __forceinline__ float scaled_value(float beta, float v) { return beta * v; }
__device__ __forceinline__ float delta_coeff(float ab, float ptil, float bv) { return __builtin_fmaf(-ab, ptil, bv); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// ------------------------------------------------- fused preprocessing numerics
//
// One fixed sequence of fp32 operations per quantity, used by every kernel:
//   softplus(x) = max(x, 0) + log1p(y),  y = 2^(-|x| log2 e)  (hardware exp2)
//                 log1p(y) = y when 1 + y rounds to 1, else log2(w) ln 2 * (y / (w - 1))
//                 with w = 1 + y rounded (the correction of the rounding of 1 + y
//                 keeps the relative error a few ulps for small y, where log2(w) alone
//                 loses up to 2^-24 / y; w - 1 is exact)
//   g           = -exp(A_log) * softplus(a + dt_bias),  exp(A_log) = 2^(A_log log2 e)
//   beta        = rcp(1 + 2^(-b log2 e))                            (hardware rcp)
//   L2 norm     : x * rsq(sumsq + eps), sumsq over leaves of 4 consecutive columns
//                 (x0*x0, then fma with x1, x2, x3), added pairwise in column order.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;

__device__ __forceinline__ float softplus_f32(float x) {
    const float y = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
    const float w = 1.f + y;
    const float l = (w == 1.f) ? y : (__builtin_amdgcn_logf(w) * kLn2) * (y / (w - 1.f));
    return __builtin_fmaxf(x, 0.f) + l;
}
__device__ __forceinline__ float gate_amplitude(float A_log) { return __builtin_amdgcn_exp2f(A_log * kLog2e); }
__device__ __forceinline__ float gate_from_logit(float amp, float dt_bias, float a) {
    return -amp * softplus_f32(a + dt_bias);
}
__device__ __forceinline__ float sigmoid_f32(float b) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-b * kLog2e));
}
__device__ __forceinline__ float sumsq4(float x0, float x1, float x2, float x3) {
    float s = x0 * x0;
    s = __builtin_fmaf(x1, x1, s);
    s = __builtin_fmaf(x2, x2, s);
    return __builtin_fmaf(x3, x3, s);
}
__device__ __forceinline__ float norm_scale(float sumsq, float eps) { return __builtin_amdgcn_rsqf(sumsq + eps); }

// x + (x of the partner lane given by a DPP control)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Tree levels above the lane-local leaves, for a row held by L lanes:
// quad_perm 1,0,3,2 (l^1), quad_perm 2,3,0,1 (l^2), row_half_mirror, row_mirror.
// Addition is commutative, so both partners compute identical bits at every level.
template <int L>
__device__ __forceinline__ float lane_sum(float x) {
    x = dpp_add<0xB1>(x);
    x = dpp_add<0x4E>(x);
    if constexpr (L >= 8) x = dpp_add<0x141>(x);
    if constexpr (L >= 16) x = dpp_add<0x140>(x);
    return x;
}

// Pairwise tree over N partial sums held by one lane, in index order.
template <int N>
__device__ __forceinline__ float leaf_tree(const float (&x)[N]) {
    if constexpr (N == 1) {
        return x[0];
    } else if constexpr (N == 2) {
        return x[0] + x[1];
    } else if constexpr (N == 4) {
        return (x[0] + x[1]) + (x[2] + x[3]);
    } else {
        static_assert(N == 8, "leaf count");
        return ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
    }
}

// Lane geometry for key dim DK with L lanes per row.
// Sum over N consecutive lanes (N a power of two up to 32, groups aligned to N),
// as a pairwise tree over lane index: every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x = dpp_add<0xB1>(x);
    if constexpr (N >= 4) x = dpp_add<0x4E>(x);
    if constexpr (N >= 8) x = dpp_add<0x141>(x);
    if constexpr (N >= 16) x = dpp_add<0x140>(x);
    if constexpr (N >= 32) x = x + __shfl_xor(x, 16);
    static_assert(N >= 1 && N <= 32 && (N & (N - 1)) == 0, "group size");
    return x;
}

template <int DK, int L>
struct Geo {
    static_assert(DK == 16 || DK == 32 || DK == 64 || DK == 128, "unsupported dk");
    static_assert(L == 4 || L == 8 || L == 16, "lanes per row");
    static constexpr int LF = (DK >= 32) ? 8 : 4;     // leaf length
    static constexpr int CPL = LF / 4;                // 4-column chunks per leaf
    static constexpr int NCH4 = DK / 16;              // chunks per l (the 4-lane view)
    static constexpr int SUB = L / 4;                 // lanes sharing one l
    static constexpr int NCH = NCH4 / SUB;            // chunks per lane
    static constexpr int C = 4 * NCH;                 // columns per lane
    static constexpr int NLEAF = NCH / CPL;           // leaves per lane
    static constexpr int RG = 64 / L;                 // row groups per wave
    static_assert(NCH >= CPL && NCH % CPL == 0, "a lane must hold whole leaves");
    // First column of this lane's chunk j is col0 + 16 j.
    __device__ static int col0(int lam) { return 16 * ((lam % SUB) * NCH) + 4 * (lam / SUB); }
    // Where 16-column chunk c of a key/query row sits in LDS.  The chunks are
    // permuted so that, at every step of a read, the L lanes of a row touch
    // distinct LDS banks (lanes differing only in lam % SUB would otherwise read
    // addresses 64*NCH bytes apart, which share banks).
    __host__ __device__ static constexpr int lds_chunk(int c) { return c ^ ((c / NCH) & (SUB - 1)); }
    // LDS float offset, inside one staged row, of this lane's chunk j.
    __device__ static int lds_col(int lam, int j) {
        return 16 * lds_chunk((lam % SUB) * NCH + j) + 4 * (lam / SUB);
    }
};

// res[r] = S[r] . x  for the R rows held by this lane (every lane of the row gets it).
template <int DK, int L, int R, int C>
__device__ __forceinline__ void row_dots(const float (&S)[R][C], const float (&x)[C], float (&res)[R]) {
    using G = Geo<DK, L>;
    static_assert(C == G::C, "columns per lane");
    float acc[R][G::NLEAF];
#pragma unroll
    for (int j = 0; j < G::NCH; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * j + e;
            const int lf = j / G::CPL;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if ((j % G::CPL) == 0 && e == 0)
                    acc[r][lf] = S[r][i] * x[i];
                else
                    acc[r][lf] = __builtin_fmaf(S[r][i], x[i], acc[r][lf]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) res[r] = lane_sum<L>(leaf_tree<G::NLEAF>(acc[r]));
}

// One token's state update and read-out for the R rows of this lane:
//   S[r][i] = fma(a, S[r][i], u[r] * kc[i])  for all i, then o[r] = S[r] . qc,
// then, when NEXT, ptil[r] = S[r] . kn (the next token's key).  Doing the whole
// update before the read-outs gives the query and next-key loads time to land.
//
// TIED writes each new state element into the register of the old one (a
// three-address v_fma_f32 with its result tied to S).  Left to itself the compiler
// uses the two-address v_fmac_f32, whose result lands in the product's register;
// where a uniform branch follows every token, the state must then be copied back
// at each join, 16 moves per token for 16 columns per lane.  Same instruction,
// same rounding, same bits: only the register assignment differs.
template <int DK, int L, int R, bool NEXT, bool TIED = false, int C>
__device__ __forceinline__ void update_sweep(float (&S)[R][C], const float (&kc)[C], const float (&qc)[C],
                                             const float (&kn)[C], float a, const float (&u)[R], float (&o)[R],
                                             float (&ptil)[R]) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float w = u[r] * kc[i];
            if constexpr (TIED)
                asm("v_fma_f32 %0, %1, %0, %2" : "+v"(S[r][i]) : "v"(a), "v"(w));
            else
                S[r][i] = __builtin_fmaf(a, S[r][i], w);
        }
    }
    row_dots<DK, L, R>(S, qc, o);
    if constexpr (NEXT) row_dots<DK, L, R>(S, kn, ptil);
}

// ------------------------------------------------------------------ io types

struct IoBf16 {
    static constexpr int VEC = 8;  // elements per 16-byte vector
    static constexpr int ESZ = 2;
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
    // Round to nearest even (v_cvt_pk_bf16_f32), the same conversion in every kernel.
    __device__ static void store1(void *base, size_t idx, float f) {
        static_cast<uint16_t *>(base)[idx] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
    }
    // VEC consecutive elements from idx (16-byte aligned), rounded as store1 does.
    __device__ static void store_vec(void *base, size_t idx, const float (&f)[VEC]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(f[2 * i])) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(f[2 * i + 1])) << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(base) + idx) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};

struct IoF32 {
    static constexpr int VEC = 4;
    static constexpr int ESZ = 4;
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
    __device__ static void store_vec(void *base, size_t idx, const float (&f)[VEC]) {
        *reinterpret_cast<float4 *>(static_cast<float *>(base) + idx) = make_float4(f[0], f[1], f[2], f[3]);
    }
};

// ------------------------------------------------------------- prefill kernel

template <int DK, class IO, int L, int R, int NW>
struct PrefillShape {
    static constexpr int TB = (NW >= 2) ? 16 : 8;    // tokens per staged block
    static constexpr int TS = TB + 1;                // staged tokens: the block and the next block's first
    static constexpr int RW = NW * (64 / L) * R;     // rows per workgroup
    static constexpr int NT = NW * 64;               // threads per workgroup
    static constexpr int KVEC = DK / IO::VEC;        // 16-byte vectors per key/query row
    static constexpr int VVEC = RW / IO::VEC;        // 16-byte vectors per value row slice
    static constexpr int KITEMS = TS * KVEC;
    static constexpr int VITEMS = TS * VVEC;
    static constexpr int KSLOTS = (KITEMS + NT - 1) / NT;
    // Query rows: only the block's own TB tokens are read (the extra staged row
    // exists for the next token's key read-out), so one slot fewer where TB rows
    // fit the workgroup's threads (4 VGPRs: 8 lanes x 2 rows then fits three waves
    // per SIMD).
    static constexpr int QITEMS = TB * KVEC;
    static constexpr int QSLOTS = (QITEMS + NT - 1) / NT;
    static constexpr int VSLOTS = (VITEMS + NT - 1) / NT;
    static constexpr int TT = L / R;                 // tokens buffered per output store
    // Guards between token steps of full blocks: 1 = every token, 0 = none.  Chosen
    // per shape from measurements on MI355X: a guard after every token keeps
    // registers (and waves per SIMD) for the 4- and 8-lane shapes; 16 lanes per row
    // is the shape for scarce rows (about one wave per SIMD), where the compiler's
    // freedom to schedule across tokens matters more than registers.
    static constexpr int GUARD = (L == 16) ? 0 : 1;
    // Waves per SIMD the register allocation must leave room for (plain instance;
    // the extended one keeps the compiler's choice).  gfx950 issues VALU
    // instructions of two waves of one SIMD in the same cycle, so throughput grows
    // with the waves a SIMD can choose from.  The 8-wave 8-lane bf16 shape fits
    // four (at most 128 VGPRs; one 8-byte spill reloaded once per token block) and
    // measured 10 % faster on equal-length batches than at three.  The other
    // shapes, fp32 io and the extended instances spill far more at 128 VGPRs.
    static constexpr int MIN_WAVES = (NW == 8 && L == 8 && R == 1 && IO::ESZ == 2) ? 4 : 1;
    static_assert(TS <= NT, "gate/beta staging needs TB+1 threads");
    static_assert(RW % IO::VEC == 0, "row slice must be whole vectors");
    static_assert(TB % TT == 0, "output flushes must align with token blocks");
};

template <int DK, class IO, int L, int R, int NW>
struct alignas(16) PrefillLds {
    using Sh = PrefillShape<DK, IO, L, R, NW>;
    float k[2][Sh::TS][DK];   // key rows, fp32, chunks permuted by Geo::lds_chunk
    float q[2][Sh::TS][DK];   // query rows, same layout
    float v[2][Sh::TS][Sh::RW];  // beta * v
    float a[2][Sh::TS];          // decay factors exp(g)
    float ab[2][Sh::TS];         // a * beta (must follow a: read as a[buf] + 2 * TS)
};

// Global -> register stage of one token block (issued early), then register -> LDS.
template <int DK, class IO, int L, int R, int NW>
struct Stager {
    using Sh = PrefillShape<DK, IO, L, R, NW>;
    using G = Geo<DK, L>;
    uint4 kr[Sh::KSLOTS];
    uint4 qr[Sh::QSLOTS];
    uint4 vr[Sh::VSLOTS];
    float vbeta[Sh::VSLOTS];  // beta of each staged value vector's token
    float gt, bt;             // g and beta of token tid (tid < TS)

    // Rows ti = 0 .. TS-1 hold token t0 + ti; tokens outside [ts, te) are zero.
    __device__ __forceinline__ void load(const PrefillParams &p, int64_t t0, int64_t ts, int64_t te, int kh, int h,
                                         int row0, int tid) {
        const uint4 zero = make_uint4(0, 0, 0, 0);
        const char *kb = static_cast<const char *>(p.k);
        const char *qb = static_cast<const char *>(p.q);
        const char *vb = static_cast<const char *>(p.v);
#pragma unroll
        for (int s = 0; s < Sh::KSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            const int ti = it / Sh::KVEC, vec = it % Sh::KVEC;
            const int64_t t = t0 + ti;
            const bool in = t >= ts && t < te;
            const size_t off = ((size_t)(t * p.hk + kh) * DK + (size_t)vec * IO::VEC) * IO::ESZ;
            kr[s] = zero;
            if (it < Sh::KITEMS && in) kr[s] = *reinterpret_cast<const uint4 *>(kb + off);
            if (s < Sh::QSLOTS) {
                qr[s] = zero;
                if (it < Sh::QITEMS && in) qr[s] = *reinterpret_cast<const uint4 *>(qb + off);
            }
        }
#pragma unroll
        for (int s = 0; s < Sh::VSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            const int ti = it / Sh::VVEC, vec = it % Sh::VVEC;
            const int64_t t = t0 + ti;
            vr[s] = zero;
            vbeta[s] = 0.f;
            if (it < Sh::VITEMS && t >= ts && t < te) {
                vr[s] = *reinterpret_cast<const uint4 *>(
                    vb + ((size_t)(t * p.hv + h) * p.dv + row0 + (size_t)vec * IO::VEC) * IO::ESZ);
                vbeta[s] = p.beta[t * p.hv + h];
            }
        }
        gt = 0.f;
        bt = 0.f;
        if (tid < Sh::TS && t0 + tid >= ts && t0 + tid < te) {
            gt = p.g[(t0 + tid) * p.hv + h];
            bt = p.beta[(t0 + tid) * p.hv + h];
        }
    }

    // Columns [col, col + 4) of a key/query row go to their permuted LDS chunk.
    __device__ static float *row_slot(float *row, int col) { return row + 16 * G::lds_chunk(col / 16) + col % 16; }

    // Row sum of squares of a key/query row: this thread's leaves of 4 columns
    // (pairwise), then the KVEC threads of the row (a pairwise tree over thread
    // index); every thread of the row gets it.  Threads past the staged items hold
    // zeros and still take part, so whole lane groups run the cross-lane levels.
    __device__ static float row_sumsq(const float (&f)[IO::VEC]) {
        float leaves[IO::VEC / 4];
#pragma unroll
        for (int x = 0; x < IO::VEC / 4; ++x) leaves[x] = sumsq4(f[4 * x], f[4 * x + 1], f[4 * x + 2], f[4 * x + 3]);
        return group_sum<Sh::KVEC>(leaf_tree<IO::VEC / 4>(leaves));
    }

    // pre: GDN_PRE_* flags; amp = exp(A_log[h]), dtb = dt_bias[h] (gated inputs only).
    __device__ __forceinline__ void store(PrefillLds<DK, IO, L, R, NW> &Ld, int buf, int tid, int pre, float eps,
                                          float amp, float dtb) const {
#pragma unroll
        for (int s = 0; s < Sh::KSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            const int ti = it / Sh::KVEC, vec = it % Sh::KVEC;
            // Without the norm, slots past the staged items (whole waves, often) skip
            // the unpacking; with it every lane of a row group must take part.
            if (!(pre & GDN_PRE_QK_L2NORM) && it >= Sh::KITEMS) continue;
            float fk[IO::VEC];
            IO::unpack(kr[s], fk);
            if (pre & GDN_PRE_QK_L2NORM) {
                const float ik = norm_scale(row_sumsq(fk), eps);
#pragma unroll
                for (int x = 0; x < IO::VEC; ++x) fk[x] = fk[x] * ik;
            }
            if (it < Sh::KITEMS) {
#pragma unroll
                for (int x = 0; x < IO::VEC; x += 4)
                    *reinterpret_cast<float4 *>(row_slot(Ld.k[buf][ti], vec * IO::VEC + x)) =
                        make_float4(fk[x], fk[x + 1], fk[x + 2], fk[x + 3]);
            }
            if (s < Sh::QSLOTS) {  // (a constant: every lane of a row group takes part)
                float fq[IO::VEC];
                IO::unpack(qr[s < Sh::QSLOTS ? s : 0], fq);
                if (pre & GDN_PRE_QK_L2NORM) {
                    const float iq = norm_scale(row_sumsq(fq), eps);
#pragma unroll
                    for (int x = 0; x < IO::VEC; ++x) fq[x] = fq[x] * iq;
                }
                if (it < Sh::QITEMS) {
#pragma unroll
                    for (int x = 0; x < IO::VEC; x += 4)
                        *reinterpret_cast<float4 *>(row_slot(Ld.q[buf][ti], vec * IO::VEC + x)) =
                            make_float4(fq[x], fq[x + 1], fq[x + 2], fq[x + 3]);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < Sh::VSLOTS; ++s) {
            const int it = tid + s * Sh::NT;
            if (it < Sh::VITEMS) {
                const int ti = it / Sh::VVEC, vec = it % Sh::VVEC;
                float f[IO::VEC];
                IO::unpack(vr[s], f);
                const float bvs = (pre & GDN_PRE_GATE_LOGITS) ? sigmoid_f32(vbeta[s]) : vbeta[s];
#pragma unroll
                for (int x = 0; x < IO::VEC; ++x) f[x] = scaled_value(bvs, f[x]);
#pragma unroll
                for (int x = 0; x < IO::VEC; x += 4)
                    *reinterpret_cast<float4 *>(&Ld.v[buf][ti][vec * IO::VEC + x]) =
                        make_float4(f[x], f[x + 1], f[x + 2], f[x + 3]);
            }
        }
        if (tid < Sh::TS) {
            const bool gated = pre & GDN_PRE_GATE_LOGITS;
            const float a = decay_factor(gated ? gate_from_logit(amp, dtb, gt) : gt);
            Ld.a[buf][tid] = a;
            Ld.ab[buf][tid] = scaled_decay(a, gated ? sigmoid_f32(bt) : bt);
        }
    }
};

// The per-token inputs one lane carries from one token to the next: the key (the
// next token's key is read during the current token's pass) and the scalars.
template <int C, int R>
struct TokRegs {
    float k[C];
    float bv[R];  // beta * v of this lane's rows
    float a, ab;  // exp(g), exp(g) * beta
};

// Work order.  Workgroups start in blockIdx order and the sequence walk is serial,
// so the longest sequences should start first (longest-processing-time-first list
// scheduling); otherwise a long sequence that starts late sets the kernel's end.
// When asked (rank_by_length, at most kMaxRankedSeqs sequences) each workgroup
// ranks the lengths itself (descending, ties by index) and takes the sequence of
// rank blockIdx.z; otherwise it takes sequence blockIdx.z.  Which sequence a
// workgroup serves never changes any result.
__device__ __forceinline__ int seq_by_length_rank(const int32_t *cu, int n_seqs, int rank, int tid, int nthreads) {
    __shared__ int32_t s_len[kMaxRankedSeqs];
    __shared__ int s_pick;
    for (int m = tid; m < n_seqs; m += nthreads) s_len[m] = cu[m + 1] - cu[m];
    __syncthreads();
    for (int m = tid; m < n_seqs; m += nthreads) {
        const int lm = s_len[m];
        int r = 0;
        for (int i = 0; i < n_seqs; ++i) {
            const int li = s_len[i];
            r += (li > lm) || (li == lm && i < m);
        }
        if (r == rank) s_pick = m;
    }
    __syncthreads();
    return s_pick;
}

// Which (sequence rank, value head, row tile) a prefill workgroup serves.
//
// Workgroups are handed to the eight XCDs round robin by id, and each XCD has its
// own L2.  All workgroups that read the same key/query rows (the `group` of one
// sequence and one key head: hv/hk value heads x tiles) are given ids that are
// equal modulo 8, so they run on one XCD and read q/k from HBM once, not once per
// XCD.  Groups are numbered rank-major, so lower ids still go to longer sequences.
// A trailing partial round of groups (fewer than 8 left) is mapped in order.
struct WorkItem {
    int rank, kh, h, tile;
};

constexpr int kXcds = 8;

__device__ __forceinline__ WorkItem work_item(const PrefillParams &p, int id) {
    const int gv = p.hv / p.hk;                 // value heads per key head
    const int gsize = gv * p.tiles;             // workgroups per group
    const int ngroups = p.n_seqs * p.hk;
    const int full = (ngroups / kXcds) * kXcds * gsize;  // workgroups in whole rounds of 8 groups
    int g, member;
    if (id < full) {
        const int xcd = id % kXcds, slot = id / kXcds;
        g = (slot / gsize) * kXcds + xcd;
        member = slot % gsize;
    } else {
        g = full / gsize + (id - full) / gsize;
        member = (id - full) % gsize;
    }
    WorkItem w;
    w.rank = g / p.hk;
    w.kh = g % p.hk;
    w.h = w.kh * gv + member / p.tiles;
    w.tile = member % p.tiles;
    return w;
}

// One workgroup = (sequence, value head, row tile), from blockIdx.x (see work_item).
// EXT compiles the extended features, state snapshots (block grid aligned to
// absolute positions) and fused preprocessing; without it the kernel carries
// none of that logic.
template <int DK, class IO, int L, int R, int NW, bool EXT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(EXT ? 1 : PrefillShape<DK, IO, L, R, NW>::MIN_WAVES)))
void gdn_prefill_kernel(PrefillParams p) {
    using Sh = PrefillShape<DK, IO, L, R, NW>;
    using G = Geo<DK, L>;
    constexpr int C = G::C, NCH = G::NCH, TB = Sh::TB, RG = G::RG, TT = Sh::TT;
    __shared__ PrefillLds<DK, IO, L, R, NW> Ld;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lam = lane % L, grp = lane / L;
    const int col0 = G::col0(lam);
    const WorkItem wi = work_item(p, blockIdx.x);
    const int h = wi.h, kh = wi.kh;
    const int row0 = wi.tile * Sh::RW;
    // (ties break by index, so the ranks are a permutation and exactly one thread picks)
    const int n = p.rank_by_length ? seq_by_length_rank(p.cu_seqlens, p.n_seqs, wi.rank, tid, NW * 64) : wi.rank;

    // Sequence bounds, clamped into [0, T] so that a malformed cu_seqlens cannot
    // send the kernel outside the buffers.
    int64_t tb = p.cu_seqlens[n], te = p.cu_seqlens[n + 1];
    tb = tb < 0 ? 0 : (tb > p.total_tokens ? p.total_tokens : tb);
    te = te < tb ? tb : (te > p.total_tokens ? p.total_tokens : te);
    const int64_t len = te - tb;

    // This lane's rows inside the tile: wrow + RG * r.
    const int wrow = wave * RG * R + grp;
    // Element offset of this lane's first state row within state slot `slot`.
    auto state_at = [&](int64_t slot) -> size_t {
        return (((size_t)slot * p.hv + h) * p.dv + row0 + wrow) * DK + col0;
    };
    auto slot_of = [&](const int32_t *idx) -> int64_t {  // -1: none
        if (!idx) return n;
        const int64_t s = idx[n];
        return (s >= 0 && s < p.pool_size) ? s : -1;
    };
    auto store_state = [&](float *base, int64_t slot, const float (&St)[R][C]) {
        float *dst = base + state_at(slot);
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < NCH; ++j)
                *reinterpret_cast<float4 *>(dst + (size_t)RG * r * DK + 16 * j) =
                    make_float4(St[r][4 * j + 0], St[r][4 * j + 1], St[r][4 * j + 2], St[r][4 * j + 3]);
        }
    };

    float S[R][C];
    {
        const int64_t src = p.h0 ? slot_of(p.src_idx) : -1;
        const float *h0row = src >= 0 ? p.h0 + state_at(src) : nullptr;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                if (h0row) x = *reinterpret_cast<const float4 *>(h0row + (size_t)RG * r * DK + 16 * j);
                S[r][4 * j + 0] = x.x; S[r][4 * j + 1] = x.y; S[r][4 * j + 2] = x.z; S[r][4 * j + 3] = x.w;
            }
        }
    }

    // Snapshots.  base = tokens already behind this sequence.  The token blocks are
    // laid on the grid of absolute positions: the first block starts at slot
    // lo0 = base % TB, so every block ends on a multiple of TB and each multiple of
    // snap_block (itself a multiple of TB) is the end of some block.  Without
    // snapshots lo0 = 0 and block b simply covers tokens [tb + b TB, tb + (b+1) TB).
    int64_t base = 0;
    if (EXT && p.snap_block > 0 && p.pos0) {
        base = p.pos0[n];
        base = base < 0 ? 0 : base;
    }
    const int lo0 = EXT ? (int)(base % TB) : 0;
    auto snapshot_after = [&](int64_t done) {  // done: tokens of this call behind the state
        const int64_t pos = base + done;
        if (!EXT || p.snap_block <= 0 || done <= 0 || pos % p.snap_block != 0) return;
        const int64_t j = pos / p.snap_block - base / p.snap_block - 1;
        if (j < 0 || j >= p.snap_per_seq) return;
        const int64_t slot = p.snap_idx[(int64_t)n * p.snap_per_seq + j];
        if (slot >= 0 && slot < p.pool_size) store_state(p.snap, slot, S);
    };

    if (len > 0) {
        const int nblk = (int)((len + lo0 + TB - 1) / TB);
        const int pre = EXT ? p.pre_flags : 0;
        const float amp = (pre & GDN_PRE_GATE_LOGITS) ? gate_amplitude(p.A_log[h]) : 0.f;
        const float dtb = ((pre & GDN_PRE_GATE_LOGITS) && p.dt_bias) ? p.dt_bias[h] : 0.f;
        Stager<DK, IO, L, R, NW> st;
        st.load(p, tb - lo0, tb, te, kh, h, row0, tid);
        st.store(Ld, 0, tid, pre, p.pre_eps, amp, dtb);
        __syncthreads();

        // LDS float offsets of this lane's chunks within a staged row.
        int lcol[NCH];
#pragma unroll
        for (int j = 0; j < NCH; ++j) lcol[j] = G::lds_col(lam, j);
        auto read_cols = [&](float (&dst)[C], const float *row) {
#pragma unroll
            for (int j = 0; j < NCH; ++j) {
                const float4 x = *reinterpret_cast<const float4 *>(row + lcol[j]);
                dst[4 * j + 0] = x.x; dst[4 * j + 1] = x.y; dst[4 * j + 2] = x.z; dst[4 * j + 3] = x.w;
            }
        };
        // The decay scalars of the current buffer are read through a VGPR pointer set
        // once per block; left alone the compiler rebuilds this uniform address (an
        // SGPR move and an add) at every token.  ab[buf] lies 2 * TS floats past a[buf].
        typedef __attribute__((address_space(3))) const float lds_f32;
        using LdsT = PrefillLds<DK, IO, L, R, NW>;
        static_assert(offsetof(LdsT, ab) == offsetof(LdsT, a) + sizeof(float) * 2 * Sh::TS, "ab follows a");
        lds_f32 *arow = (lds_f32 *)&Ld.a[0][0];
        asm volatile("" : "+v"(arow));
        auto fetch = [&](TokRegs<C, R> &X, int buf, int ti) {
            read_cols(X.k, Ld.k[buf][ti]);
#pragma unroll
            for (int r = 0; r < R; ++r) X.bv[r] = Ld.v[buf][ti][wrow + RG * r];
            X.a = arow[ti];
            X.ab = arow[ti + 2 * Sh::TS];
        };

        // Outputs are kept in registers and stored TT tokens at a time: lane lam
        // keeps token (lam % TT) of its row lam / TT.
        const int my_slot = lam % TT, my_r = lam / TT;
        const size_t out_row = (size_t)h * p.dv + row0 + wrow + RG * my_r;
        float obuf = 0.f;
        // The training forward also keeps p_t = S_{t-1} k_t (ptil before the step) for
        // the backward, buffered and stored like the outputs.
        const bool save = EXT && p.save_p != nullptr;
        float pbuf = 0.f;

        // Slot ti is processed with cur = A when ti is even and cur = B when odd, so
        // the first token (slot lo0) starts in both.
        TokRegs<C, R> A, B;
        float ptil[R];
        fetch(A, 0, lo0);
        if constexpr (EXT) B = A;
        row_dots<DK, L, R>(S, A.k, ptil);

        for (int blk = 0; blk < nblk; ++blk) {
            const int buf = blk & 1;
            // Slot ti of this block is token t0 + ti; slots [lo, nt) are tokens of the
            // sequence (lo > 0 only in a first block that starts mid-grid).
            const int lo = (EXT && blk == 0) ? lo0 : 0;
            const int64_t t0 = tb - lo0 + (int64_t)blk * TB;
            if (blk + 1 < nblk) st.load(p, t0 + TB, tb, te, kh, h, row0, tid);
            const int nt = (int)((te - t0) < TB ? (te - t0) : TB);
            arow = (lds_f32 *)&Ld.a[buf][0];
            asm volatile("" : "+v"(arow));

            // cur holds token ti; nxt receives token ti + 1 (staged row ti + 1 <= TB).
            auto step = [&](TokRegs<C, R> &cur, TokRegs<C, R> &nxt, int ti) {
#ifdef GDN_TOKEN_SCHED_FENCE
                __builtin_amdgcn_sched_barrier(0);
#endif
                float u[R], o[R];
#pragma unroll
                for (int r = 0; r < R; ++r) u[r] = delta_coeff(cur.ab, ptil[r], cur.bv[r]);
                if constexpr (EXT) {
                    if (save) {
                        float pv = ptil[0];
#pragma unroll
                        for (int r = 1; r < R; ++r)
                            if (my_r == r) pv = ptil[r];
                        if (my_slot == ti % TT) pbuf = pv;
                    }
                }
                float qc[C];
                read_cols(qc, Ld.q[buf][ti]);
                fetch(nxt, buf, ti + 1);
                update_sweep<DK, L, R, true, Sh::GUARD == 1>(S, cur.k, qc, nxt.k, cur.a, u, o, ptil);
                float ov = o[0];
#pragma unroll
                for (int r = 1; r < R; ++r)
                    if (my_r == r) ov = o[r];
                if (my_slot == ti % TT) obuf = ov;
                if (ti % TT == TT - 1 && (!EXT || ti - (TT - 1) + my_slot >= lo)) {
                    const size_t oi = (size_t)(t0 + ti - (TT - 1) + my_slot) * p.hv * p.dv + out_row;
                    IO::store1(p.out, oi, obuf);
                    if constexpr (EXT)
                        if (save) p.save_p[oi] = pbuf;
                }
            };

            // Full token blocks are fully unrolled.  The last block of a sequence
            // may be partial (and a first block may start mid-grid); uniform guards
            // skip the missing slots.  Where guards also sit between steps of full
            // blocks they bound how far the compiler hoists work across tokens, which
            // trades some in-wave overlap for fewer registers (more waves per SIMD);
            // the best trade depends on the shape (measured on MI355X), see Sh::GUARD.
            if constexpr (Sh::GUARD == 0) {
                if (lo == 0 && nt == TB) {
#pragma unroll
                    for (int ti = 0; ti < TB; ti += 2) {
                        step(A, B, ti);
                        step(B, A, ti + 1);
                    }
                } else {
#pragma unroll
                    for (int ti = 0; ti < TB; ti += 2) {
                        if (ti >= lo && ti < nt) step(A, B, ti);
                        if (ti + 1 >= lo && ti + 1 < nt) step(B, A, ti + 1);
                    }
                }
            } else {
#pragma unroll
                for (int ti = 0; ti < TB; ti += 2) {
                    if (ti >= lo && ti < nt) step(A, B, ti);
                    if (ti + 1 >= lo && ti + 1 < nt) step(B, A, ti + 1);
                }
            }
            const int rem = nt % TT;  // tokens kept but not yet stored (partial block only)
            if (rem != 0 && my_slot < rem && (!EXT || nt - rem + my_slot >= lo)) {
                const size_t oi = (size_t)(t0 + nt - rem + my_slot) * p.hv * p.dv + out_row;
                IO::store1(p.out, oi, obuf);
                if constexpr (EXT)
                    if (save) p.save_p[oi] = pbuf;
            }
            if constexpr (EXT) snapshot_after(t0 + nt - tb);

            if (blk + 1 < nblk) st.store(Ld, buf ^ 1, tid, pre, p.pre_eps, amp, dtb);
            __syncthreads();
        }
    }

    if (p.hT) {
        const int64_t dst = slot_of(p.dst_idx);
        if (dst >= 0) store_state(p.hT, dst, S);
    }
}

// -------------------------------------------------------------- decode kernel

// One workgroup = (batch row b = blockIdx.z, value head h = blockIdx.y, row tile blockIdx.x).
// Four lanes per row: the state streams once through registers.
template <int DK, class IO, int R, int NW, bool EXT>
__global__ __launch_bounds__(NW * 64) void gdn_decode_kernel(DecodeParams p) {
    constexpr int L = 4;
    using G = Geo<DK, L>;
    constexpr int C = G::C, RG = G::RG;
    constexpr int RW = NW * RG * R;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lam = lane % L, grp = lane / L;
    const int col0 = G::col0(lam);
    const int b = blockIdx.z, h = blockIdx.y;
    const int row0 = blockIdx.x * RW;
    const int kh = h / (p.hv / p.hk);
    const int wrow = wave * RG * R + grp;
    const size_t orow = ((size_t)b * p.hv + h) * p.dv + row0 + wrow;

    const int slot = p.state_idx ? p.state_idx[b] : b;
    if (slot < 0 || slot >= p.pool_size) {  // padding row: zero output, no state access
        if (lam < R) IO::store1(p.out, orow + RG * lam, 0.f);
        return;
    }
    float *st = p.pool + (((size_t)slot * p.hv + h) * p.dv + row0 + wrow) * DK;

    float S[R][C];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int j = 0; j < G::NCH; ++j) {
            const float4 x = *reinterpret_cast<const float4 *>(st + (size_t)RG * r * DK + col0 + 16 * j);
            S[r][4 * j + 0] = x.x; S[r][4 * j + 1] = x.y; S[r][4 * j + 2] = x.z; S[r][4 * j + 3] = x.w;
        }
    }
    float kx[C], qx[C];
    const size_t qk0 = ((size_t)b * p.hk + kh) * DK + col0;
#pragma unroll
    for (int j = 0; j < G::NCH; ++j) {
        const float4 k4 = IO::load4(p.k, qk0 + 16 * j);
        const float4 q4 = IO::load4(p.q, qk0 + 16 * j);
        kx[4 * j + 0] = k4.x; kx[4 * j + 1] = k4.y; kx[4 * j + 2] = k4.z; kx[4 * j + 3] = k4.w;
        qx[4 * j + 0] = q4.x; qx[4 * j + 1] = q4.y; qx[4 * j + 2] = q4.z; qx[4 * j + 3] = q4.w;
    }
    const int pre = EXT ? p.pre_flags : 0;
    if (pre & GDN_PRE_QK_L2NORM) {
        // The staging order of the prefill kernel: leaves of 4 columns (this lane
        // holds leaf 4j + lam of chunk j), pairs across lam, then chunks pairwise.
        float ck[G::NCH], cq[G::NCH];
#pragma unroll
        for (int j = 0; j < G::NCH; ++j) {
            ck[j] = group_sum<4>(sumsq4(kx[4 * j], kx[4 * j + 1], kx[4 * j + 2], kx[4 * j + 3]));
            cq[j] = group_sum<4>(sumsq4(qx[4 * j], qx[4 * j + 1], qx[4 * j + 2], qx[4 * j + 3]));
        }
        const float ik = norm_scale(leaf_tree<G::NCH>(ck), p.pre_eps);
        const float iq = norm_scale(leaf_tree<G::NCH>(cq), p.pre_eps);
#pragma unroll
        for (int i = 0; i < C; ++i) {
            kx[i] = kx[i] * ik;
            qx[i] = qx[i] * iq;
        }
    }
    float a, beta;
    if (pre & GDN_PRE_GATE_LOGITS) {
        const float amp = gate_amplitude(p.A_log[h]);
        const float dtb = p.dt_bias ? p.dt_bias[h] : 0.f;
        a = decay_factor(gate_from_logit(amp, dtb, p.g[(size_t)b * p.hv + h]));
        beta = sigmoid_f32(p.beta[(size_t)b * p.hv + h]);
    } else {
        a = decay_factor(p.g[(size_t)b * p.hv + h]);
        beta = p.beta[(size_t)b * p.hv + h];
    }
    const float ab = scaled_decay(a, beta);

    float ptil[R], u[R], o[R];
    row_dots<DK, L, R>(S, kx, ptil);
#pragma unroll
    for (int r = 0; r < R; ++r) u[r] = delta_coeff(ab, ptil[r], scaled_value(beta, IO::load1(p.v, orow + RG * r)));
    update_sweep<DK, L, R, false>(S, kx, qx, kx, a, u, o, ptil);

#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int j = 0; j < G::NCH; ++j)
            *reinterpret_cast<float4 *>(st + (size_t)RG * r * DK + col0 + 16 * j) =
                make_float4(S[r][4 * j + 0], S[r][4 * j + 1], S[r][4 * j + 2], S[r][4 * j + 3]);
    }
    float ov = o[0];
#pragma unroll
    for (int r = 1; r < R; ++r)
        if (lam == r) ov = o[r];
    if (lam < R) IO::store1(p.out, orow + RG * lam, ov);
}

// ------------------------------------------------------------ launch helpers

template <int DK, class IO, int L, int R, int NW>
hipError_t launch_prefill_t(const PrefillParams &p, hipStream_t s) {
    constexpr int RW = NW * (64 / L) * R;
    PrefillParams q = p;
    q.tiles = p.dv / RW;
    dim3 grid((unsigned)q.tiles * p.hv * p.n_seqs), block(NW * 64);
    void *args[] = {&q};
    const bool ext = p.snap_block > 0 || p.pre_flags != 0 || p.save_p != nullptr;
    const void *fn = ext ? reinterpret_cast<const void *>(&gdn_prefill_kernel<DK, IO, L, R, NW, true>)
                         : reinterpret_cast<const void *>(&gdn_prefill_kernel<DK, IO, L, R, NW, false>);
    return hipLaunchKernel(fn, grid, block, args, 0, s);
}

template <int DK, class IO, int R, int NW>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t s) {
    constexpr int RW = NW * 16 * R;
    dim3 grid(p.dv / RW, p.hv, p.batch), block(NW * 64);
    void *args[] = {const_cast<DecodeParams *>(&p)};
    const void *fn = p.pre_flags != 0 ? reinterpret_cast<const void *>(&gdn_decode_kernel<DK, IO, R, NW, true>)
                                      : reinterpret_cast<const void *>(&gdn_decode_kernel<DK, IO, R, NW, false>);
    return hipLaunchKernel(fn, grid, block, args, 0, s);
}

}  // namespace gdn
