// gdn_chunked.hip -- the chunked form of the gated delta rule with a decode that
// replays it (gdn_fwd_chunked).
//
// The page "Defending Against the Training-Inference Numeric Mismatch in RL
// (Especially Linear Attention)" (section 3.2) makes prefill and decode agree by
// running the recurrence token by token everywhere.  The summary of "Finish RL
// Training Faster: Bitwise-Consistent, High-Performance, Agent-Driven" (section
// "Consistency has several layers") describes the other way: a chunked prefill
// whose decode replays its computation order.  That needs chunk boundaries that do
// not move with the serving split (the bitwise-parity post on linear attention,
// "Why linear attention is the next wall").  This file is that design.
//
// Chunks are the 16-token stretches of a sequence at positions 16c .. 16c + 15.
// Within a chunk, with S0 the state at its start, G_m = g_0 + ... + g_m (cumulative
// log decay, slot order), Gam_m = exp(G_m) and Gam_{m,r} = exp(G_m - G_r):
//
//     w_m = S0 k_m,   z_m = S0 q_m                                  (row dots)
//     u_m = beta_m (v_m - Gam_m w_m) - sum_{r<m} beta_m Gam_{m,r} (k_m . k_r) u_r
//     o_m = Gam_m z_m + sum_{s<=m} Gam_{m,s} (q_m . k_s) u_s
//     at the chunk's end:  S = Gam_15 S0 + sum_{s} Gam_{15,s} u_s k_s^T
//
// which is the recurrence S_m = a_m S_{m-1} + u_m k_m^T, o_m = S_m q_m written from
// the chunk's start (S_m = Gam_m S0 + sum_{s<=m} Gam_{m,s} u_s k_s^T).  Every
// quantity of token m depends only on S0 and the chunk's tokens up to m, each with
// one fixed sequence of fp32 operations.  The state between calls is therefore S0
// plus the open chunk's k, u and G (and its token count), and any split of a
// sequence into calls, a decode step of one token included, gives the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.hpp"
#include "gdn_kernels.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

constexpr int kCk = kChunkLen;       // tokens per chunk (16)
constexpr int kChLanes = 8;          // lanes per state row
constexpr int kChWaves = 4;
constexpr int kChRows = kChWaves * (64 / kChLanes);  // rows per workgroup (32)
constexpr int kChThreads = kChWaves * 64;

template <int DK>
struct alignas(16) ChunkLds {
    float k[kCk][DK];       // keys of the chunk's slots (cached or new)
    float q[kCk][DK];       // queries of the new slots
    float v[kCk][kChRows];  // values of this tile's rows
    float ckk[kCk][kCk];    // beta_m Gam_{m,r} (k_m . k_r), r < m
    float cqk[kCk][kCk];    // Gam_{m,s} (q_m . k_s), s <= m
    float cst[kCk];         // Gam_{15,s}: weights of the chunk-end state update
    float G[kCk];           // cumulative log decay of each slot
    float gam[kCk];         // Gam_m
    float beta[kCk];
};

// LDS position (in 4-float chunks) of lane lam's j-th 4-column chunk of a key or
// query row.  With 16 columns per lane (dk = 128) the j-th chunks of lanes lam and
// lam + 4 would share banks, so those lanes keep their chunks in a rotated order.
template <int DK>
__device__ __forceinline__ int ch_slot(int lam, int j) {
    constexpr int CH = DK / kChLanes / 4;
    if constexpr (CH == 4) return lam * CH + ((j + (lam >> 2)) & 3);
    else return lam * CH + j;
}

// This lane's C columns of an LDS key/query row (chunk offsets lch).
template <int C>
__device__ __forceinline__ void load_cols(float (&dst)[C], const float *row, const int (&lch)[C / 4]) {
#pragma unroll
    for (int j = 0; j < C / 4; ++j) {
        const float4 x = *reinterpret_cast<const float4 *>(row + lch[j]);
        dst[4 * j] = x.x; dst[4 * j + 1] = x.y; dst[4 * j + 2] = x.z; dst[4 * j + 3] = x.w;
    }
}

template <int C>
__device__ __forceinline__ float chunk_lane_dot(const float (&x)[C], const float (&y)[C]) {
    constexpr int K = C >= 16 ? 4 : (C >= 8 ? 2 : 1);
    float acc[K];
#pragma unroll
    for (int c = 0; c < K; ++c) acc[c] = x[c] * y[c];
#pragma unroll
    for (int c = K; c < C; ++c) acc[c % K] = __builtin_fmaf(x[c], y[c], acc[c % K]);
    if constexpr (K == 1) return acc[0];
    else if constexpr (K == 2) return acc[0] + acc[1];
    else return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// One workgroup = (sequence n, value head h, tile of 32 state rows).
template <int DK, class IO>
__global__ __launch_bounds__(kChThreads) void gdn_chunked_kernel(ChunkedParams p) {
    constexpr int C = DK / kChLanes;
    __shared__ ChunkLds<DK> Ld;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lam = lane % kChLanes, grp = lane / kChLanes;
    const int tiles = p.dv / kChRows;
    const int tile = blockIdx.x % tiles;
    const int h = (blockIdx.x / tiles) % p.hv;
    const int n = blockIdx.x / (tiles * p.hv);
    const int G_ = p.hv / p.hk;
    const int kh = h / G_;
    const int lrow = wave * (64 / kChLanes) + grp;
    const int row = tile * kChRows + lrow;
    const int col0 = lam * C;
    int lch[C / 4];  // LDS float offsets of this lane's column chunks in a key/query row
#pragma unroll
    for (int j = 0; j < C / 4; ++j) lch[j] = 4 * ch_slot<DK>(lam, j);
    // where 4-column chunk c4 of a row is kept (the inverse view of lch, for staging)
    auto stage_off = [](int c4) { return 4 * ch_slot<DK>((4 * c4) / C, ((4 * c4) % C) / 4); };

    int64_t tb = p.cu_seqlens[n], te = p.cu_seqlens[n + 1];
    tb = tb < 0 ? 0 : (tb > p.total_tokens ? p.total_tokens : tb);
    te = te < tb ? tb : (te > p.total_tokens ? p.total_tokens : te);
    const int64_t len = te - tb;

    // incoming state: S0 rows, the open chunk's count, u (this row), k and G
    int m0 = 0;
    if (p.in_count) {
        m0 = p.in_count[n];
        m0 = m0 < 0 ? 0 : (m0 >= kCk ? kCk - 1 : m0);
    }
    const size_t sbase = (((size_t)n * p.hv + h) * p.dv + row) * DK + col0;
    float X[C];
#pragma unroll
    for (int c = 0; c < C; c += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.in_S) x = *reinterpret_cast<const float4 *>(p.in_S + sbase + c);
        X[c] = x.x; X[c + 1] = x.y; X[c + 2] = x.z; X[c + 3] = x.w;
    }
    float ureg[kCk];
#pragma unroll
    for (int m = 0; m < kCk; ++m) {
        ureg[m] = 0.f;
        if (m < m0) ureg[m] = p.in_u[(((size_t)n * kCk + m) * p.hv + h) * p.dv + row];
    }
    for (int idx = tid; idx < m0 * (DK / 4); idx += kChThreads) {
        const int m = idx / (DK / 4), c4 = idx % (DK / 4);
        *reinterpret_cast<float4 *>(&Ld.k[m][stage_off(c4)]) =
            *reinterpret_cast<const float4 *>(p.in_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + 4 * c4);
    }
    if (tid < m0) Ld.G[tid] = p.in_G[((size_t)n * kCk + tid) * p.hv + h];
    __syncthreads();

    int ms = m0;            // first open slot of the current chunk
    int64_t done = 0;       // tokens of this call processed
    while (done < len) {
        const int take = (int)((len - done) < (int64_t)(kCk - ms) ? (len - done) : (kCk - ms));
        const int me = ms + take;                // slots [ms, me) are new tokens
        const int64_t t_of_slot0 = tb + done - ms;  // token index of slot 0

        // ---- stage the new slots
        for (int idx = tid; idx < take * (DK / 4); idx += kChThreads) {
            const int m = ms + idx / (DK / 4), c4 = idx % (DK / 4);
            const size_t qk = ((size_t)(t_of_slot0 + m) * p.hk + kh) * DK + 4 * c4;
            *reinterpret_cast<float4 *>(&Ld.k[m][stage_off(c4)]) = IO::load4(p.k, qk);
            *reinterpret_cast<float4 *>(&Ld.q[m][stage_off(c4)]) = IO::load4(p.q, qk);
        }
        for (int idx = tid; idx < take * kChRows; idx += kChThreads) {
            const int m = ms + idx / kChRows, r = idx % kChRows;
            Ld.v[m][r] = IO::load1(p.v, ((size_t)(t_of_slot0 + m) * p.hv + h) * p.dv + tile * kChRows + r);
        }
        if (wave == 0) {  // cumulative log decay, added in slot order (lane j holds g of slot ms + j)
            const float gj = lane < take ? p.g[(size_t)(t_of_slot0 + ms + lane) * p.hv + h] : 0.f;
            float acc = ms > 0 ? Ld.G[ms - 1] : 0.f;
            for (int j = 0; j < take; ++j) {
                acc = acc + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gj), j));
                if (lane == j) Ld.G[ms + j] = acc;
            }
        }
        if (tid < take) Ld.beta[ms + tid] = p.beta[(size_t)(t_of_slot0 + ms + tid) * p.hv + h];
        __syncthreads();

        // ---- coefficient tables of the new slots: each entry's dot is spread over the
        // 8 lanes of a group (C columns each, then the lane tree), 32 groups per
        // workgroup; entry e = (m, r) of the (take x 16) table.
        for (int e0 = 0; e0 < take * kCk; e0 += kChThreads / kChLanes) {
            const int e = e0 + tid / kChLanes;
            const int m = ms + e / kCk, r = e % kCk;
            const bool live = e < take * kCk && r <= m;
            float kv[C], km[C], qm[C];
            load_cols<C>(kv, Ld.k[live ? r : 0], lch);
            load_cols<C>(km, Ld.k[live ? m : 0], lch);
            load_cols<C>(qm, Ld.q[live ? m : 0], lch);
            const float dkk = lane_sum<kChLanes>(chunk_lane_dot<C>(kv, km));
            const float dqk = lane_sum<kChLanes>(chunk_lane_dot<C>(kv, qm));
            if (live && lam == 0) {
                const float gm = decay_factor(Ld.G[m] - Ld.G[r]);
                if (r < m) Ld.ckk[m][r] = Ld.beta[m] * gm * dkk;
                Ld.cqk[m][r] = gm * dqk;
            }
        }
        if (tid < take) Ld.gam[ms + tid] = decay_factor(Ld.G[ms + tid]);
        if (me == kCk && tid < kCk) Ld.cst[tid] = decay_factor(Ld.G[kCk - 1] - Ld.G[tid]);
        __syncthreads();

        // ---- the new slots, in order (unrolled over the 16 slots, guarded)
#pragma unroll
        for (int m = 0; m < kCk; ++m) {
            if (m < ms || m >= me) continue;
            float km[C], qm[C];
            load_cols<C>(km, Ld.k[m], lch);
            load_cols<C>(qm, Ld.q[m], lch);
            const float w = lane_sum<kChLanes>(chunk_lane_dot<C>(X, km));
            const float z = lane_sum<kChLanes>(chunk_lane_dot<C>(X, qm));
            float u = Ld.beta[m] * (Ld.v[m][lrow] - Ld.gam[m] * w);
#pragma unroll
            for (int r = 0; r < m; ++r) u = __builtin_fmaf(-Ld.ckk[m][r], ureg[r], u);
            ureg[m] = u;
            float o = Ld.gam[m] * z;
#pragma unroll
            for (int s = 0; s <= m; ++s) o = __builtin_fmaf(Ld.cqk[m][s], ureg[s], o);
            if (lam == 0) IO::store1(p.out, ((size_t)(t_of_slot0 + m) * p.hv + h) * p.dv + row, o);
        }

        // ---- chunk complete: fold it into the state
        if (me == kCk) {
            const float g15 = Ld.gam[kCk - 1];
#pragma unroll
            for (int c = 0; c < C; ++c) X[c] = g15 * X[c];
#pragma unroll
            for (int s = 0; s < kCk; ++s) {
                const float cs = Ld.cst[s] * ureg[s];
                float ks[C];
                load_cols<C>(ks, Ld.k[s], lch);
#pragma unroll
                for (int c = 0; c < C; ++c) X[c] = __builtin_fmaf(cs, ks[c], X[c]);
            }
        }
        done += take;
        ms = me == kCk ? 0 : me;
        __syncthreads();
    }

    // ---- outgoing state: S0 of the open chunk, its count, k, u and G
#pragma unroll
    for (int c = 0; c < C; c += 4)
        *reinterpret_cast<float4 *>(p.out_S + sbase + c) = make_float4(X[c], X[c + 1], X[c + 2], X[c + 3]);
    const int mo = ms;  // tokens in the open chunk after this call
#pragma unroll
    for (int m = 0; m < kCk; ++m)
        if (m < mo && lam == 0) p.out_u[(((size_t)n * kCk + m) * p.hv + h) * p.dv + row] = ureg[m];
    if (tile == 0 && h % G_ == 0)
        for (int idx = tid; idx < mo * (DK / 4); idx += kChThreads) {
            const int m = idx / (DK / 4), c4 = idx % (DK / 4);
            *reinterpret_cast<float4 *>(p.out_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + 4 * c4) =
                *reinterpret_cast<const float4 *>(&Ld.k[m][stage_off(c4)]);
        }
    if (tile == 0 && tid < mo) p.out_G[((size_t)n * kCk + tid) * p.hv + h] = Ld.G[tid];
    if (tile == 0 && h == 0 && tid == 0) p.out_count[n] = mo;
}

template <class IO>
hipError_t chunked_io(const ChunkedParams &p, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)p.n_seqs * p.hv * (p.dv / kChRows)));
    switch (p.dk) {
        case 64: hipLaunchKernelGGL((gdn_chunked_kernel<64, IO>), grid, dim3(kChThreads), 0, s, p); break;
        case 128: hipLaunchKernelGGL((gdn_chunked_kernel<128, IO>), grid, dim3(kChThreads), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunked(const ChunkedParams &p, int io_dtype, hipStream_t s) {
    return io_dtype == GDN_BF16 ? chunked_io<IoBf16>(p, s) : chunked_io<IoF32>(p, s);
}

}  // namespace gdn
