// gdn_chunked.hip -- the chunked form of the gated delta rule on the matrix cores,
// with a decode that replays it (gdn_fwd_chunked).
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
// Within a chunk, with S0 the state at its start and a_m = exp(g_m):
//
//     Gam_{m,r} = a_m a_{m-1} ... a_{r+1}   (r < m; 1 for r = m),   Gam_m = Gam_{m,0} a_0
//     P_m = S0 k_m,   Z_m = S0 q_m,   R_m = beta_m (v_m - Gam_m P_m)
//     A[m][r] = beta_m Gam_{m,r} (k_m . k_r)  (r < m),   T = (I + A)^-1   (unit lower triangular)
//     U = T R            (so u_m = R_m - sum_{r<m} A[m][r] u_r)
//     O = Gam Z + B U,   B[m][s] = Gam_{m,s} (q_m . k_s)  (s <= m)
//     at the chunk's end:  S = Gam_15 S0 + sum_s Gam_{15,s} u_s k_s^T
//
// which is the recurrence S_m = a_m S_{m-1} + u_m k_m^T, o_m = S_m q_m written from
// the chunk's start (the WY form of the delta rule's products).  Every product with
// the state, U, O, the chunk-end update and the key/query Gram tiles run as fp32 MFMA
// (v_mfma_f32_16x16x4f32, fp32 accumulation); T comes from a per-column forward
// substitution in a separate, fully parallel kernel, so a chunk's walk has no serial
// vector chain.
//
// Fixed arithmetic.  Every quantity is one fixed sequence of operations whatever the
// batch, the launch or the split of a sequence into calls:
//   * an MFMA dot over dk is the chain of instructions t = 0 .. dk/16-1, i = 0 .. 3,
//     instruction (t, i) adding the products of columns 16t + 4g + i, g = 0..3; an
//     output element depends only on its own row and column of the operands, so a
//     decode step that holds one token in its tile forms that token's bits;
//   * a product over the chunk's tokens (U, O, the chunk-end update) is the chain of
//     instructions r = 0..3, instruction r adding the tokens 4g + r, g = 0..3.  T and
//     B are zero above the diagonal, so a later token enters an earlier token's
//     result only as exact zero products; a decode step holds zeros for the tokens it
//     has not seen, the sums agree, and +0 is added to U and O so that an exactly
//     zero result has one sign.  (A NaN or infinity in a token therefore reaches the
//     earlier tokens of its chunk, 0 x NaN being NaN; finite inputs replay exactly.)
//   * Gam products, the coefficient tables and T are fixed-order fp32 chains.
// The state between calls is S0 plus the open chunk's keys, R rows, decay factors
// and betas (and its token count); a decode step runs the same two kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.hpp"
#include "gdn_mfma.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

constexpr int kCk = kChunkLen;   // tokens per chunk (16)

// Clamped sequence bounds and chunk bookkeeping shared by both kernels.
struct SeqChunks {
    int64_t tb, len;  // first token of the sequence in this call, tokens in this call
    int c0;           // tokens already in the open chunk (from the incoming state)
    int nch;          // chunks this call touches
    int64_t base;     // first workspace slot of the sequence
};

__device__ __forceinline__ int64_t clamp_tok(int64_t x, int64_t T) { return x < 0 ? 0 : (x > T ? T : x); }

__device__ __forceinline__ SeqChunks seq_chunks(const ChunkedParams &p, int n) {
    SeqChunks s;
    // (no cu_seqlens: one token per sequence, sequence n's token is token n)
    s.tb = p.cu_seqlens ? clamp_tok(p.cu_seqlens[n], p.total_tokens) : n;
    int64_t te = p.cu_seqlens ? clamp_tok(p.cu_seqlens[n + 1], p.total_tokens) : n + 1;
    te = te < s.tb ? s.tb : te;
    s.len = te - s.tb;
    int c0 = p.in_count ? p.in_count[n] : 0;
    s.c0 = c0 < 0 ? 0 : (c0 > kCk - 1 ? kCk - 1 : c0);
    s.nch = s.len > 0 ? (int)((s.c0 + s.len + kCk - 1) / kCk) : 0;
    s.base = chunk_slot_base(s.tb, n);
    return s;
}

// ------------------------------------------------------------------- prep kernel
//
// One workgroup (256 threads) per (workspace slot, key head).  It stages the chunk's
// keys (cached and new) and new queries, forms the Gram tiles K K^T and Q K^T with
// MFMA (waves 0 and 1), then for each value head of the key head writes the record
// the main kernel reads: A[m][r] = (beta_m Gam_{m,r}) (k_m . k_r) for r < m,
// B[m][s] = Gam_{m,s} (q_m . k_s) for s <= m (rows of the chunk's new tokens only),
// Gam_m, the chunk-end weights Gam_{15,s} and the decay factors a_m.
// With BW (the backward's forward walk) the record is kChunkRecBwd floats and also
// holds Gam_{m,s} for s <= m and Gam_{m,s} (k_m . k_s) for s < m.
template <int DK, class IO, bool BW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(7))) void gdn_chunk_prep_kernel(ChunkedParams p) {
    constexpr int NT = DK / 16;
    constexpr int REC = BW ? kChunkRecBwd : kChunkRec;
    constexpr int KP = DK + 4;  // padded LDS row
    __shared__ __align__(16) float Ks[kCk][KP];  // (16-byte aligned: accessed as float4)
    __shared__ __align__(16) float Qs[kCk][KP];
    __shared__ float kap[kCk][kCk + 1];
    __shared__ float xi[kCk][kCk + 1];

    const int kh = blockIdx.y;
    const int tid = threadIdx.x;
    // The sequence owning this slot: the last n with base(n) <= slot.  Without
    // cu_seqlens (one token per sequence) the grid has one workgroup per sequence,
    // whose only chunk takes slot base(n).
    int64_t slot;
    int n;
    if (p.cu_seqlens) {
        slot = blockIdx.x;
        int lo = 0, hi = p.n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (chunk_slot_base(clamp_tok(p.cu_seqlens[mid], p.total_tokens), mid) <= slot)
                lo = mid;
            else
                hi = mid - 1;
        }
        n = lo;
    } else {
        n = blockIdx.x;
        slot = chunk_slot_base(n, n);
    }
    const SeqChunks sc = seq_chunks(p, n);
    const int64_t j = slot - sc.base;
    if (j < 0 || j >= sc.nch || slot >= p.ws_slots) return;  // uniform over the workgroup
    const int m0 = j == 0 ? sc.c0 : 0;
    const int64_t left = sc.c0 + sc.len - kCk * j;
    const int m1 = left < kCk ? (int)left : kCk;
    const int64_t t0 = sc.tb + kCk * j - sc.c0;  // token index of chunk position 0

    // One round of reads: the chunk's key rows (cached and new) and new query rows,
    // and the decay factors and betas of every value head of this key head.
    constexpr int kMaxG = 16;  // value heads per key head handled per workgroup (host-checked)
    __shared__ float decs[kMaxG][kCk], bets[kMaxG][kCk];
    const int G = p.hv / p.hk;
    for (int it = tid; it < kCk * (DK / 4); it += 256) {
        const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
        if (m < m1) {
            if (m < m0) {  // cached key of the open chunk (fp32)
                kv = *reinterpret_cast<const float4 *>(p.in_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + c);
            } else {
                const size_t e = ((size_t)(t0 + m) * p.hk + kh) * DK + c;
                kv = IO::load4(p.k, e);
                qv = IO::load4(p.q, e);
            }
        }
        *reinterpret_cast<float4 *>(&Ks[m][c]) = kv;
        *reinterpret_cast<float4 *>(&Qs[m][c]) = qv;
    }
    for (int it = tid; it < G * kCk; it += 256) {
        const int gi = it / kCk, m = it % kCk, h = kh * G + gi;
        float a = 0.f, b = 0.f;
        if (m < m1) {
            if (m < m0) {
                a = p.in_a[((size_t)n * kCk + m) * p.hv + h];
                b = p.in_b[((size_t)n * kCk + m) * p.hv + h];
            } else {
                a = decay_factor(p.g[(size_t)(t0 + m) * p.hv + h]);
                b = p.beta[(size_t)(t0 + m) * p.hv + h];
            }
        }
        decs[gi][m] = a;
        bets[gi][m] = b;
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63, x = lane & 15, g = lane >> 4;
    if (wave < 2) {
        // wave 0: kap = K K^T, wave 1: xi = Q K^T  (A rows from K or Q, B rows from K)
        const float(*Arows)[KP] = wave == 0 ? Ks : Qs;
        f4 acc = f4_zero();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 a4 = *reinterpret_cast<const float4 *>(&Arows[x][16 * t + 4 * g]);
            const float4 b4 = *reinterpret_cast<const float4 *>(&Ks[x][16 * t + 4 * g]);
            acc = mfma_16x16x4(a4.x, b4.x, acc);
            acc = mfma_16x16x4(a4.y, b4.y, acc);
            acc = mfma_16x16x4(a4.z, b4.z, acc);
            acc = mfma_16x16x4(a4.w, b4.w, acc);
        }
        float(*dst)[kCk + 1] = wave == 0 ? kap : xi;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[4 * g + r][x] = acc[r];
    }

    __shared__ float Am[kCk][kCk + 1];
    const int m = tid / kCk, r = tid % kCk;
    for (int gi = 0; gi < G; ++gi) {
        const int h = kh * G + gi;
        __syncthreads();  // Gram tiles written; Am free again
        const float *dec = decs[gi], *bet = bets[gi];
        // Gam_{m,r} = a_m a_{m-1} ... a_{r+1}, left to right (1 for r >= m); the
        // factors come from registers, s descending, each taken when r < s <= m
        float dreg[kCk];
#pragma unroll
        for (int s = 0; s < kCk; ++s) dreg[s] = dec[s];
        float gmr = 1.f;
#pragma unroll
        for (int s = kCk - 1; s >= 0; --s) gmr = (s <= m && s > r) ? gmr * dreg[s] : gmr;
        const bool row = m < m1;
        Am[m][r] = (row && r < m) ? (bet[m] * gmr) * kap[m][r] : 0.f;
        const bool newrow = m >= m0 && m < m1;
        float *rec = p.ws + ((size_t)slot * p.hv + h) * REC;
        rec[kRecB + m * kCk + r] = (newrow && r <= m) ? gmr * xi[m][r] : 0.f;
        if constexpr (BW) {
            rec[kRecGm + m * kCk + r] = (row && r <= m) ? gmr : 0.f;
            rec[kRecAb + m * kCk + r] = (row && r < m) ? gmr * kap[m][r] : 0.f;
        }
        if (r == 0) rec[kRecGam + m] = row ? gmr * dreg[0] : 0.f;
        if (m == kCk - 1) rec[kRecD + r] = gmr;
        if (r == 0) {
            rec[kRecDecay + m] = dec[m];
            rec[kRecBeta + m] = bet[m];
        }
        __syncthreads();
        // T = (I + A)^-1 by columns: lane k of wave 0 walks column k,
        // T[m][k] = -(sum_{r=k}^{m-1} A[m][r] T[r][k]) (r ascending), T[k][k] = 1.
        if (tid < kCk) {
            const int k = tid;
            float col[kCk];
#pragma unroll
            for (int mm = 0; mm < kCk; ++mm) {
                float acc = 0.f;
#pragma unroll
                for (int rr = 0; rr < mm; ++rr)
                    if (rr >= k) acc = __builtin_fmaf(Am[mm][rr], col[rr], acc);
                col[mm] = mm < k ? 0.f : (mm == k ? 1.f : -acc);
                if (mm >= m1) col[mm] = 0.f;
                rec[kRecT + mm * kCk + k] = col[mm];
            }
        }
    }
}

// ------------------------------------------------------------------- main kernel
//
// One workgroup = (sequence, value head, 16 state rows) with W waves (1, 2 or 4).
// The dk columns are cut into four quarters; wave w owns quarters [4w/W, 4(w+1)/W)
// of the state tile, held transposed as MFMA accumulator tiles: lane l = x + 16 g
// holds S[row0 + x][16 t + 4 g + c] in component c of tile t.  Token-by-row tiles
// (P, Z, R, U, O) use the MFMA output layout: lane x + 16 g holds token 4 g + c, row x.
//
// P and Z are defined as ((X_0 + X_1) + (X_2 + X_3)), X_q the MFMA chain over the
// tiles of quarter q.  A wave forms the partials of its quarters; with W > 1 they
// meet in LDS and every wave adds the four in that order, so every W gives the same
// bits.  R, U and O are then formed alike in every wave (wave 0 stores them); each
// wave folds its own tiles at a chunk's end.
//
// Every global read of a chunk (new keys, queries, values, betas and the record's T
// and B rows, Gam and chunk-end weights) is sent out when the previous chunk starts
// its products, into registers, with rows outside the chunk clamped to a valid row
// and zeroed after the load (no branch per load).

// What one chunk needs from global memory, per lane of a W-wave workgroup.  The lean
// form stages the queries in LDS like the keys instead of holding them as operands.
template <int DK, class IO, int W, bool LEAN>
struct ChunkFetch {
    static constexpr int KIT = kCk * DK / 4 / (64 * W);  // 4-element key items per lane (LDS staging)
    static constexpr int OT = DK / 16 / W;               // state tiles owned by one wave
    typename Raw4<IO>::T kr[LEAN ? 1 : KIT];  // key rows for LDS: item tid + 64 W s
    typename Raw4<IO>::T qa[LEAN ? 1 : OT];   // query operand: token x, columns of the wave's tiles
    uint32_t v[4];                  // value bits (row x) of tokens 4 g + c
    float4 b;                       // their betas (from the record)
    float4 trow, brow;              // T[x][4 g ..] and B[x][4 g ..]
    float4 gam, dw;                 // Gam_{4 g + c} and chunk-end weights Gam_{15, 4 g + c}
    float g15;                      // Gam_15
};

// MODE 0: the chunked form.  MODE 2 (lean): the same arithmetic, instruction for
// instruction, for calls of a few tokens per sequence (a decode step): no read-ahead
// of the next chunk, queries and the chunk-end update's key operands read from LDS
// when used, so that four waves fit on a SIMD and their memory latencies overlap.
// MODE 1: the forward walk of the chunked backward.  No outputs: the state at each
// chunk's start goes to the checkpoints, x = v - Gam P to xv, and every chunk folds
// (a sequence's last, partial chunk with the weights of its last token, so that the
// final state is hT), which gives the partial sums of <dhT, hT>.
template <int DK, class IO, int W, int MODE>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(MODE == 2 ? 3 : 1)))
void gdn_chunk_main_kernel(ChunkedParams p) {
    constexpr bool BW = MODE == 1, LEAN = MODE == 2;
    constexpr int REC = BW ? kChunkRecBwd : kChunkRec;
    constexpr int NT = DK / 16;
    constexpr int KP = DK + 4;
    constexpr int OT = NT / W;       // tiles per wave
    constexpr int QT = NT / 4;       // tiles per quarter
    constexpr int OQ = 4 / W;        // quarters per wave
    using CF = ChunkFetch<DK, IO, W, LEAN>;
    using RW = Raw4<IO>;
    static_assert(NT % 4 == 0 && OT * W == NT, "tiles");
    __shared__ __align__(16) float Ks[kCk][KP];         // the chunk's keys, fp32 (accessed as float4)
    __shared__ __align__(16) float Qs[LEAN ? kCk : 1][KP];  // (lean) the chunk's queries
    __shared__ float4 Xch[W > 1 ? 8 : 1][64];           // P and Z partials of the four quarters

    // (the wave index as a uniform value, so that tests on it are scalar branches)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int x = lane & 15, g = lane >> 4;
    const int tiles = p.dv / 16;
    // Workgroups are handed to the eight XCDs round robin by id.  The ones that read
    // the same keys and queries (one sequence and key head: hv/hk value heads x
    // tiles) get ids equal modulo 8, so they share one XCD's L2; groups are numbered
    // rank-major so that lower ids still go to longer sequences.
    int rank, h, tile;
    {
        const int G = p.hv / p.hk, gsize = G * tiles;
        const int ngroups = p.n_seqs * p.hk;
        const int full = (ngroups / 8) * 8 * gsize;
        const int id = blockIdx.x;
        int grp, member;
        if (id < full) {
            const int xcd = id % 8, slot = id / 8;
            grp = (slot / gsize) * 8 + xcd;
            member = slot % gsize;
        } else {
            grp = full / gsize + (id - full) / gsize;
            member = (id - full) % gsize;
        }
        rank = grp / p.hk;
        h = (grp % p.hk) * G + member / tiles;
        tile = member % tiles;
    }
    const int n = p.rank_by_length ? seq_by_length_rank(p.cu_seqlens, p.n_seqs, rank, tid, 64 * W) : rank;
    const int kh = h / (p.hv / p.hk);
    const int row0 = tile * 16;
    const int t_first = wave * OT;   // first state tile of this wave
    const SeqChunks sc = seq_chunks(p, n);
    const bool inplace = p.inplace != 0;
    const size_t krow = (size_t)p.hk * DK, vrow = (size_t)p.hv * p.dv;

    // state tiles of this wave
    f4 S[OT];
    {
        const float *src = p.in_S ? p.in_S + (((size_t)n * p.hv + h) * p.dv + row0 + x) * DK : nullptr;
#pragma unroll
        for (int t = 0; t < OT; ++t) {
            S[t] = f4_zero();
            if (src) {
                const float4 v4 = *reinterpret_cast<const float4 *>(src + 16 * (t_first + t) + 4 * g);
                S[t] = f4{v4.x, v4.y, v4.z, v4.w};
            }
        }
    }

    int nch = sc.nch;  // chunks with a workspace slot (all of them for a well-formed cu_seqlens)
    if (sc.base + nch > p.ws_slots) nch = (int)(p.ws_slots - sc.base > 0 ? p.ws_slots - sc.base : 0);
    // chunk j: positions [m0, m1) are this call's tokens, token of position 0 is t0
    auto geom = [&](int j, int &m0, int &m1, int64_t &t0) {
        m0 = j == 0 ? sc.c0 : 0;
        const int64_t left = sc.c0 + sc.len - (int64_t)kCk * j;
        m1 = left < kCk ? (int)left : kCk;
        t0 = sc.tb + (int64_t)kCk * j - sc.c0;
    };
    auto clampm = [](int m, int lo, int hi) { return m < lo ? lo : (m >= hi ? hi - 1 : m); };
    // byte offset of this lane's value (row x, token 4 g) within a chunk's value rows
    const uint32_t v_lane = (uint32_t)(4 * g) * (uint32_t)(vrow * IO::ESZ) + (uint32_t)(row0 + x) * IO::ESZ;
    // (j is clamped to the last chunk, so that a read past it repeats that chunk's
    // reads instead of needing a branch; nch >= 1 whenever this is called)
    auto fetch = [&](CF &F, int j_) {
        const int j = j_ < nch ? j_ : nch - 1;
        int m0, m1;
        int64_t t0;
        geom(j, m0, m1, t0);
        // uniform bases of this chunk; per-lane offsets in bytes (a chunk spans 16 tokens)
        constexpr uint32_t E = IO::ESZ;
        const char *kb = static_cast<const char *>(p.k) + ((size_t)t0 * p.hk + kh) * DK * E;
        const char *qb = static_cast<const char *>(p.q) + ((size_t)t0 * p.hk + kh) * DK * E;
        const char *vb = static_cast<const char *>(p.v) + ((size_t)t0 * p.hv + h) * p.dv * E;
        const uint32_t krow_b = (uint32_t)krow * E, vrow_b = (uint32_t)vrow * E;
#pragma unroll
        for (int s = 0; s < CF::KIT; ++s) {
            const int it = tid + 64 * W * s;
            const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
            if constexpr (!LEAN) F.kr[s] = RW::load_at(kb, (uint32_t)clampm(m, m0, m1) * krow_b + (uint32_t)c * E);
        }
        if constexpr (!BW && !LEAN) {
            const uint32_t qoff = (uint32_t)clampm(x, m0, m1) * krow_b + (uint32_t)(16 * t_first + 4 * g) * E;
#pragma unroll
            for (int t = 0; t < OT; ++t) F.qa[t] = RW::load_at(qb, qoff + 16u * t * E);
        }
        if (!LEAN && m0 == 0 && m1 == kCk) {  // a full chunk: token 4 g + c at the lane's offset plus c rows
#pragma unroll
            for (int c = 0; c < 4; ++c) F.v[c] = RW::load1_at(vb, v_lane + (uint32_t)c * vrow_b);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t tm = (uint32_t)clampm(4 * g + c, m0, m1);
                F.v[c] = RW::load1_at(vb, tm * vrow_b + (uint32_t)(row0 + x) * E);
            }
        }
        const char *rec = reinterpret_cast<const char *>(p.ws + ((size_t)(sc.base + j) * p.hv + h) * REC);
        // the betas of tokens 4 g .. 4 g + 3 as the prep kernel put them in the record
        // (the same values; zero past the chunk's end)
        F.b = *reinterpret_cast<const float4 *>(rec + 4u * (kRecBeta + 4 * g));
        F.trow = *reinterpret_cast<const float4 *>(rec + 4u * (kRecT + x * kCk + 4 * g));
        F.gam = *reinterpret_cast<const float4 *>(rec + 4u * (kRecGam + 4 * g));
        if constexpr (BW) {
            // the fold weights of the chunk's last token: Gam_{m1-1, s} and Gam_{m1-1}
            F.dw = *reinterpret_cast<const float4 *>(rec + 4u * (kRecGm + (m1 - 1) * kCk + 4 * g));
            F.g15 = *reinterpret_cast<const float *>(rec + 4u * (kRecGam + m1 - 1));
        } else {
            F.brow = *reinterpret_cast<const float4 *>(rec + 4u * (kRecB + x * kCk + 4 * g));
            F.dw = *reinterpret_cast<const float4 *>(rec + 4u * (kRecD + 4 * g));
            F.g15 = *reinterpret_cast<const float *>(rec + 4u * (kRecGam + kCk - 1));
        }
    };

    int last_m0 = sc.c0, mo = sc.c0;
    bool folded = false;
    // R rows of the open chunk (tokens 4 g + c, row x): cached ones first
    float Rkeep[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (4 * g + c < sc.c0 && p.in_r) Rkeep[c] = p.in_r[(((size_t)n * kCk + 4 * g + c) * p.hv + h) * p.dv + row0 + x];

    // The chunked form (MODE 0) reads two chunks ahead into alternating register sets,
    // which it has the registers for; the walk keeps one set and four waves per SIMD.
    constexpr int AHEAD = MODE == 0 ? 2 : 1;
    CF FA, FB;
    if (!LEAN && nch > 0) fetch(FA, 0);
    if (AHEAD == 2 && nch > 1) fetch(FB, 1);
    for (int j0 = 0; j0 < nch; j0 += AHEAD) {
#pragma unroll
        for (int half = 0; half < AHEAD; ++half) {
            const int j = j0 + half;
            if (j >= nch) break;
            CF &F = half ? FB : FA;  // (resolved at compile time)
            int m0, m1;
            int64_t t0;
            geom(j, m0, m1, t0);
            const bool full = m1 == kCk;
            if constexpr (LEAN) fetch(F, j);

            // keys into LDS (cached keys of a resumed chunk only when it closes here), the
            // rest of this chunk's reads into working registers, then the next chunk's reads
            if constexpr (LEAN) {
                // zeros in the rows outside this call's tokens, and those rows read
                // straight into LDS (the same values and zeros as below; no registers held
                // for the rows; each row written by one loop only)
                const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int s = 0; s < CF::KIT; ++s) {
                    const int it = tid + 64 * W * s;
                    const int m = it / (DK / 4);
                    if (m < m0 || m >= m1) {
                        *reinterpret_cast<float4 *>(&Ks[m][4 * (it % (DK / 4))]) = z4;
                        *reinterpret_cast<float4 *>(&Qs[m][4 * (it % (DK / 4))]) = z4;
                    }
                }
                const char *kb = static_cast<const char *>(p.k) + ((size_t)t0 * p.hk + kh) * DK * IO::ESZ;
                const char *qb = static_cast<const char *>(p.q) + ((size_t)t0 * p.hk + kh) * DK * IO::ESZ;
                const uint32_t krow_b = (uint32_t)krow * IO::ESZ;
                for (int it = m0 * (DK / 4) + tid; it < m1 * (DK / 4); it += 64 * W) {
                    const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
                    const uint32_t off = (uint32_t)m * krow_b + (uint32_t)c * IO::ESZ;
                    const typename RW::T kw = RW::load_at(kb, off), qw = RW::load_at(qb, off);
                    *reinterpret_cast<float4 *>(&Ks[m][c]) = RW::widen(kw);
                    *reinterpret_cast<float4 *>(&Qs[m][c]) = RW::widen(qw);
                }
            } else {
#pragma unroll
                for (int s = 0; s < CF::KIT; ++s) {
                    const int it = tid + 64 * W * s;
                    const int m = it / (DK / 4);
                    *reinterpret_cast<float4 *>(&Ks[m][4 * (it % (DK / 4))]) = RW::widen(RW::keep(F.kr[s], m >= m0 && m < m1));
                }
            }
            if (m0 > 0 && full) {
                for (int it = tid; it < m0 * (DK / 4); it += 64 * W) {
                    const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
                    *reinterpret_cast<float4 *>(&Ks[m][c]) =
                        *reinterpret_cast<const float4 *>(p.in_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + c);
                }
            }
            float4 qv[BW || LEAN ? 1 : OT];
            if constexpr (!BW && !LEAN) {
#pragma unroll
                for (int t = 0; t < OT; ++t) qv[t] = RW::widen(RW::keep(F.qa[t], x >= m0 && x < m1));
            }
            float vb[4], bb[4], vraw[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool on = 4 * g + c >= m0 && 4 * g + c < m1;
                bb[c] = on ? (c == 0 ? F.b.x : c == 1 ? F.b.y : c == 2 ? F.b.z : F.b.w) : 0.f;
                vraw[c] = on ? RW::widen1(F.v[c]) : 0.f;
                vb[c] = bb[c] * vraw[c];
            }
            const float4 trow = F.trow, brow = F.brow, gam = F.gam, dwv = F.dw;
            const float g15 = F.g15;
            if constexpr (!LEAN) fetch(F, j + AHEAD);
            if constexpr (BW) {
                // the state at this chunk's start (stored after the next chunk's reads, so
                // that waiting for those does not wait for these)
                // (tile-major: [dk / 16 column tiles][dv rows][16 columns], so that each store
                // instruction writes 1 KB in one piece; nontemporal, read back only by the
                // reverse walk)
                float *dst = p.ck + ((size_t)(sc.base + j) * p.hv + h) * p.dv * DK + (size_t)(row0 + x) * 16 + 4 * g;
#pragma unroll
                for (int t = 0; t < OT; ++t)
                    __builtin_nontemporal_store(S[t], reinterpret_cast<f4 *>(dst + (size_t)(t_first + t) * p.dv * 16));
            }
            lds_barrier();

            // partial products of this wave's quarters
            f4 Pq[OQ], Zq[OQ];
#pragma unroll
            for (int q = 0; q < OQ; ++q) {
                Pq[q] = f4_zero();
                Zq[q] = f4_zero();
                // (lean: operands read from LDS one quarter at a time, not all up front)
                if constexpr (LEAN) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int tt = 0; tt < QT; ++tt) {
                    const int t = q * QT + tt;  // the wave's tile index
                    const float4 ka = *reinterpret_cast<const float4 *>(&Ks[x][16 * (t_first + t) + 4 * g]);
                    if constexpr (BW) {
                        Pq[q] = mfma_16x16x4(ka.x, S[t][0], Pq[q]);
                        Pq[q] = mfma_16x16x4(ka.y, S[t][1], Pq[q]);
                        Pq[q] = mfma_16x16x4(ka.z, S[t][2], Pq[q]);
                        Pq[q] = mfma_16x16x4(ka.w, S[t][3], Pq[q]);
                    } else {
                        const float4 qa = LEAN ? *reinterpret_cast<const float4 *>(&Qs[x][16 * (t_first + t) + 4 * g])
                                               : qv[LEAN ? 0 : t];
                        Pq[q] = mfma_16x16x4(ka.x, S[t][0], Pq[q]);
                        Zq[q] = mfma_16x16x4(qa.x, S[t][0], Zq[q]);
                        Pq[q] = mfma_16x16x4(ka.y, S[t][1], Pq[q]);
                        Zq[q] = mfma_16x16x4(qa.y, S[t][1], Zq[q]);
                        Pq[q] = mfma_16x16x4(ka.z, S[t][2], Pq[q]);
                        Zq[q] = mfma_16x16x4(qa.z, S[t][2], Zq[q]);
                        Pq[q] = mfma_16x16x4(ka.w, S[t][3], Pq[q]);
                        Zq[q] = mfma_16x16x4(qa.w, S[t][3], Zq[q]);
                    }
                }
            }
            f4 P4[4], Z4[4];
            if constexpr (W == 1) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    P4[q] = Pq[q];
                    Z4[q] = Zq[q];
                }
            } else {
#pragma unroll
                for (int q = 0; q < OQ; ++q) {
                    const int gq = wave * OQ + q;
                    Xch[gq][lane] = make_float4(Pq[q][0], Pq[q][1], Pq[q][2], Pq[q][3]);
                    if constexpr (!BW) Xch[4 + gq][lane] = make_float4(Zq[q][0], Zq[q][1], Zq[q][2], Zq[q][3]);
                }
                lds_barrier();
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 a4 = Xch[q][lane];
                    P4[q] = f4{a4.x, a4.y, a4.z, a4.w};
                    if constexpr (!BW) {
                        const float4 b4 = Xch[4 + q][lane];
                        Z4[q] = f4{b4.x, b4.y, b4.z, b4.w};
                    } else {
                        Z4[q] = f4_zero();
                    }
                }
            }
            f4 P, Z;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                P[c] = (P4[0][c] + P4[1][c]) + (P4[2][c] + P4[3][c]);
                Z[c] = (Z4[0][c] + Z4[1][c]) + (Z4[2][c] + Z4[3][c]);
            }

            // the chunk-end update's key operands (K^T tiles of this wave), read early
            const bool fold = BW || full;
            float kt[LEAN ? 1 : OT][4];
            if (!LEAN && fold) {
#pragma unroll
                for (int t = 0; t < OT; ++t)
#pragma unroll
                    for (int c = 0; c < 4; ++c) kt[t][c] = Ks[4 * g + c][16 * (t_first + t) + x];
            }

            // R_m = fma(-(beta_m Gam_m), P_m, beta_m v_m) for this call's tokens, cached R
            // for the chunk's earlier tokens, 0 for tokens not reached yet
            const float gm[4] = {gam.x, gam.y, gam.z, gam.w};
            f4 R, OC, X4;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int m = 4 * g + c;
                const bool on = m >= m0 && m < m1;
                if constexpr (BW) {
                    // x = v - Gam P (kept for the reverse walk; zero past the chunk's end), R = beta x
                    X4[c] = on ? __builtin_fmaf(-gm[c], P[c], vraw[c]) : 0.f;
                    R[c] = bb[c] * X4[c];
                } else {
                    const float fresh = __builtin_fmaf(-(bb[c] * gm[c]), P[c], vb[c]);
                    R[c] = on ? fresh : (m < m0 ? Rkeep[c] : 0.f);
                    Rkeep[c] = on ? fresh : Rkeep[c];
                    OC[c] = gm[c] * Z[c];
                }
            }

            if constexpr (BW) {
                // x of the chunk's 16 tokens on the tile's 16 rows: [row][token] per (chunk
                // slot, value head, row tile), so that lane (x, g) holds tokens 4 g .. 4 g + 3
                // of row x as one 16-byte piece and wave 0 writes the tile's 1 KB in one store
                const auto xrsrc = buf_rsrc(p.xv + (((size_t)(sc.base + j) * p.hv + h) * p.dv + row0) * kCk, 1024u);
                buf_store_f4_nt(xrsrc, wave == 0 ? (uint32_t)(x * kCk + 4 * g) * 4u : kDropped, X4);
            }

            // U = T R, then O = Gam Z + B U (instruction c adds the tokens 4 g + c)
            f4 U = f4_zero();
            U = mfma_16x16x4(trow.x, R[0], U);
            U = mfma_16x16x4(trow.y, R[1], U);
            U = mfma_16x16x4(trow.z, R[2], U);
            U = mfma_16x16x4(trow.w, R[3], U);
#pragma unroll
            for (int c = 0; c < 4; ++c) U[c] = U[c] + 0.f;
            if constexpr (!BW) {
            // this chunk's rows of the outputs, as buffer stores that every lane issues
            // (kDropped where there is nothing to write)
            const uint32_t col_b = (uint32_t)(h * p.dv + row0 + x);
            const auto orsrc = buf_rsrc(static_cast<const char *>(p.out) + (size_t)t0 * vrow * IO::ESZ,
                                        (uint32_t)(m1 * vrow * IO::ESZ));
            f4 O = OC;
            O = mfma_16x16x4(brow.x, U[0], O);
            O = mfma_16x16x4(brow.y, U[1], O);
            O = mfma_16x16x4(brow.z, U[2], O);
            O = mfma_16x16x4(brow.w, U[3], O);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int m = 4 * g + c;
                const bool st = wave == 0 && m >= m0 && m < m1;
                buf_store1<IO>(orsrc, st ? ((uint32_t)m * (uint32_t)vrow + col_b) * (uint32_t)IO::ESZ : kDropped, O[c] + 0.f);
            }
            }

            // chunk complete: S^T = Gam_15 S^T + K^T W, W[s][row] = Gam_{15,s} u_s (own tiles)
            if (fold) {
                const float w0 = dwv.x * U[0], w1 = dwv.y * U[1], w2 = dwv.z * U[2], w3 = dwv.w * U[3];
#pragma unroll
                for (int t = 0; t < OT; ++t) {
                    f4 C = f4{g15 * S[t][0], g15 * S[t][1], g15 * S[t][2], g15 * S[t][3]};
                    float k4[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) k4[c] = LEAN ? Ks[4 * g + c][16 * (t_first + t) + x] : kt[LEAN ? 0 : t][c];
                    C = mfma_16x16x4(k4[0], w0, C);
                    C = mfma_16x16x4(k4[1], w1, C);
                    C = mfma_16x16x4(k4[2], w2, C);
                    C = mfma_16x16x4(k4[3], w3, C);
                    S[t] = C;
                }
                folded = true;
            }
            last_m0 = full ? 0 : m0;
            mo = full ? 0 : m1;
            lds_barrier();  // Ks and Xch are refilled by the next chunk
        }
    }

    if constexpr (BW) {
        // partial sums of <dhT, hT>, one per dk quarter of the tile (so the same for
        // every W), each in a fixed lane order
        if (p.dhT) {
            const float *src = p.dhT + (((size_t)n * p.hv + h) * p.dv + row0 + x) * DK;
#pragma unroll
            for (int q = 0; q < OQ; ++q) {
                float acc = 0.f;
#pragma unroll
                for (int tt = 0; tt < QT; ++tt) {
                    const int t = q * QT + tt;
                    const float4 d4 = *reinterpret_cast<const float4 *>(src + 16 * (t_first + t) + 4 * g);
                    acc = __builtin_fmaf(S[t][0], d4.x, acc);
                    acc = __builtin_fmaf(S[t][1], d4.y, acc);
                    acc = __builtin_fmaf(S[t][2], d4.z, acc);
                    acc = __builtin_fmaf(S[t][3], d4.w, acc);
                }
                acc = sum16(acc);
                acc = acc + __shfl_xor(acc, 16, 64);
                acc = acc + __shfl_xor(acc, 32, 64);
                if (lane == 0) p.hdot[(((size_t)n * p.hv + h) * tiles + tile) * 4 + wave * OQ + q] = acc;
            }
        }
        return;
    }
    // ---- outgoing state: S0 of the open chunk (each wave its tiles), then, from wave
    // 0, its R rows, keys, decays, betas and count
    if (!inplace || folded) {
        float *dst = p.out_S + (((size_t)n * p.hv + h) * p.dv + row0 + x) * DK;
#pragma unroll
        for (int t = 0; t < OT; ++t)
            *reinterpret_cast<float4 *>(dst + 16 * (t_first + t) + 4 * g) =
                make_float4(S[t][0], S[t][1], S[t][2], S[t][3]);
    }
    if (wave != 0) return;
    const int first = inplace ? last_m0 : 0;  // rows already in place need no write
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int m = 4 * g + c;
        if (m >= first && m < mo) p.out_r[(((size_t)n * kCk + m) * p.hv + h) * p.dv + row0 + x] = Rkeep[c];
    }
    if (tile == 0) {
        // Rows [first, mo) of the open chunk.  With a chunk processed in this call, its
        // record holds every row's decay factor and beta (the cached ones copied by the
        // prep kernel); its rows below last_m0 are cached keys (only when no chunk
        // boundary was crossed), the others this call's keys.  With none, all cached.
        const bool any = nch > 0;
        const int64_t t0 = sc.tb + (int64_t)kCk * (any ? nch - 1 : 0) - sc.c0;  // token of the last chunk's slot 0
        if (lane >= first && lane < mo) {
            const float *rec = p.ws + ((size_t)(sc.base + nch - 1) * p.hv + h) * kChunkRec;
            const size_t e = ((size_t)n * kCk + lane) * p.hv + h;
            p.out_a[e] = any ? rec[kRecDecay + lane] : p.in_a[e];
            p.out_b[e] = any ? rec[kRecBeta + lane] : p.in_b[e];
        }
        if (h % (p.hv / p.hk) == 0) {
            for (int it = lane; it < kCk * (DK / 4); it += 64) {
                const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
                if (m < first || m >= mo) continue;
                float4 kv;
                if (any && m >= last_m0)
                    kv = IO::load4(p.k, ((size_t)(t0 + m) * p.hk + kh) * DK + c);
                else
                    kv = *reinterpret_cast<const float4 *>(p.in_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + c);
                *reinterpret_cast<float4 *>(p.out_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + c) = kv;
            }
            if (h == 0 && lane == 0) p.out_count[n] = mo;
        }
    }
}

// A one-token-per-sequence call without cu_seqlens (sequence n's token is row n): one
// wave per (sequence, value head) forms the chunk's tables itself (no prep launch,
// the prep kernel's operations in its order), then walks that head's 16-row state
// tiles, reading the next tile's state while the current one computes.  Each tile's
// arithmetic is the main kernel's for a one-token call, instruction for instruction
// (P, Z, R, U, O and the chunk-end update as above), so the bits are the main
// kernel's, and a prefill's.
template <int DK, class IO>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void gdn_chunk_decode_kernel(ChunkedParams p) {
    constexpr int NT = DK / 16, KP = DK + 4, QT = NT / 4;
    using RW = Raw4<IO>;
    __shared__ __align__(16) float Ks[kCk][KP];
    __shared__ __align__(16) float Qrow[DK];  // the token's query (the only query row used)
    __shared__ float decs[kCk], bets[kCk], gams[kCk], dws[kCk];
    __shared__ float kap[kCk][kCk + 1], xi[kCk][kCk + 1], Tm[kCk][kCk + 1];
    const int lane = threadIdx.x, x = lane & 15, g = lane >> 4;
    const int tiles = p.dv / 16;
    const int G = p.hv / p.hk;
    int n, h;
    {
        // value heads of one key head get ids equal modulo 8 (one XCD, one L2)
        const int ngroups = p.n_seqs * p.hk;
        const int full = (ngroups / 8) * 8 * G;
        const int id = blockIdx.x;
        int grp, member;
        if (id < full) {
            const int xcd = id % 8, slot = id / 8;
            grp = (slot / G) * 8 + xcd;
            member = slot % G;
        } else {
            grp = full / G + (id - full) / G;
            member = (id - full) % G;
        }
        n = grp / p.hk;
        h = (grp % p.hk) * G + member;
    }
    const int kh = h / G;
    int c0 = p.in_count ? p.in_count[n] : 0;
    c0 = c0 < 0 ? 0 : (c0 > kCk - 1 ? kCk - 1 : c0);
    const int m0 = c0, m1 = c0 + 1;
    const bool full = m1 == kCk;
    const bool inplace = p.inplace != 0;
    const size_t vrow = (size_t)p.hv * p.dv;
    const float bt = p.beta[(size_t)n * p.hv + h];

    // The chunk's tables, formed here with the prep kernel's operations in its order:
    // keys (cached, then the token's) in LDS with zero rows after them, the decay
    // factors and betas, the Gram tiles K K^T and Q K^T (MFMA chains), Gam, A, B, the
    // chunk-end weights, and T = (I + A)^-1 by columns.  (Query rows other than the
    // token's are zero in the prep kernel; they only reach rows no result reads.)
    for (int it = lane; it < kCk * (DK / 4); it += 64) {
        const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m < m0)
            kv = *reinterpret_cast<const float4 *>(p.in_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + c);
        else if (m == m0)
            kv = RW::widen(RW::load(p.k, ((size_t)n * p.hk + kh) * DK + c));
        *reinterpret_cast<float4 *>(&Ks[m][c]) = kv;
    }
    for (int it = lane; it < DK / 4; it += 64)
        *reinterpret_cast<float4 *>(&Qrow[4 * it]) = RW::widen(RW::load(p.q, ((size_t)n * p.hk + kh) * DK + 4 * it));
    if (lane < kCk) {
        const int m = lane;
        float a = 0.f, b = 0.f;
        if (m < m0) {
            a = p.in_a[((size_t)n * kCk + m) * p.hv + h];
            b = p.in_b[((size_t)n * kCk + m) * p.hv + h];
        } else if (m == m0) {
            a = decay_factor(p.g[(size_t)n * p.hv + h]);
            b = bt;
        }
        decs[m] = a;
        bets[m] = b;
    }
    lds_barrier();
    {
        f4 ak = f4_zero(), aq = f4_zero();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 b4 = *reinterpret_cast<const float4 *>(&Ks[x][16 * t + 4 * g]);
            const float4 q4 = x == m0 ? *reinterpret_cast<const float4 *>(&Qrow[16 * t + 4 * g])
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
            ak = mfma_16x16x4(b4.x, b4.x, ak);
            aq = mfma_16x16x4(q4.x, b4.x, aq);
            ak = mfma_16x16x4(b4.y, b4.y, ak);
            aq = mfma_16x16x4(q4.y, b4.y, aq);
            ak = mfma_16x16x4(b4.z, b4.z, ak);
            aq = mfma_16x16x4(q4.z, b4.z, aq);
            ak = mfma_16x16x4(b4.w, b4.w, ak);
            aq = mfma_16x16x4(q4.w, b4.w, aq);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            kap[4 * g + r][x] = ak[r];
            xi[4 * g + r][x] = aq[r];
        }
    }
    lds_barrier();
    // entries (m, r), four per lane; A over kap and B over xi in place (each entry is
    // read and written by its own lane)
    for (int e = lane; e < kCk * kCk; e += 64) {
        const int m = e / kCk, r = e % kCk;
        float dreg[kCk];
#pragma unroll
        for (int s = 0; s < kCk; ++s) dreg[s] = decs[s];
        float gmr = 1.f;
#pragma unroll
        for (int s = kCk - 1; s >= 0; --s) gmr = (s <= m && s > r) ? gmr * dreg[s] : gmr;
        const bool row = m < m1;
        kap[m][r] = (row && r < m) ? (bets[m] * gmr) * kap[m][r] : 0.f;  // A
        const bool newrow = m >= m0 && m < m1;
        xi[m][r] = (newrow && r <= m) ? gmr * xi[m][r] : 0.f;            // B
        if (r == 0) gams[m] = row ? gmr * dreg[0] : 0.f;
        if (m == kCk - 1) dws[r] = gmr;
    }
    lds_barrier();
    if (lane < kCk) {
        const int k = lane;
        float col[kCk];
#pragma unroll
        for (int mm = 0; mm < kCk; ++mm) {
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < mm; ++rr)
                if (rr >= k) acc = __builtin_fmaf(kap[mm][rr], col[rr], acc);
            col[mm] = mm < k ? 0.f : (mm == k ? 1.f : -acc);
            if (mm >= m1) col[mm] = 0.f;
            Tm[mm][k] = col[mm];
        }
    }
    lds_barrier();
    const float4 trow = make_float4(Tm[x][4 * g], Tm[x][4 * g + 1], Tm[x][4 * g + 2], Tm[x][4 * g + 3]);
    const float4 brow = make_float4(xi[x][4 * g], xi[x][4 * g + 1], xi[x][4 * g + 2], xi[x][4 * g + 3]);
    const float gm[4] = {gams[4 * g], gams[4 * g + 1], gams[4 * g + 2], gams[4 * g + 3]};
    const float4 dwv = make_float4(dws[4 * g], dws[4 * g + 1], dws[4 * g + 2], dws[4 * g + 3]);
    const float g15 = gams[kCk - 1];

    // tile 0's state, value and cached R rows; then each tile reads the next one's
    f4 Sn[NT];
    float vn, rn[4];
    auto read_tile = [&](int tile) {
        const int row0 = tile * 16;
        const float *src = p.in_S ? p.in_S + (((size_t)n * p.hv + h) * p.dv + row0 + x) * DK : nullptr;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            Sn[t] = f4_zero();
            if (src) {
                const float4 v4 = *reinterpret_cast<const float4 *>(src + 16 * t + 4 * g);
                Sn[t] = f4{v4.x, v4.y, v4.z, v4.w};
            }
        }
        vn = IO::load1(p.v, (size_t)n * vrow + (size_t)h * p.dv + row0 + x);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            rn[c] = 0.f;
            if (4 * g + c < c0 && p.in_r) rn[c] = p.in_r[(((size_t)n * kCk + 4 * g + c) * p.hv + h) * p.dv + row0 + x];
        }
    };
    read_tile(0);
    const int first = inplace ? (full ? 0 : m0) : 0;  // rows of the open chunk to write (R, a, b, k)
    const int mo = full ? 0 : m1;
    for (int tile = 0; tile < tiles; ++tile) {
        const int row0 = tile * 16;
        f4 S[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) S[t] = Sn[t];
        const float vv = vn;
        float Rkeep[4] = {rn[0], rn[1], rn[2], rn[3]};
        if (tile + 1 < tiles) read_tile(tile + 1);

        f4 Pq[4], Zq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            Pq[q] = f4_zero();
            Zq[q] = f4_zero();
            __builtin_amdgcn_sched_barrier(0);  // operands read one quarter at a time
#pragma unroll
            for (int tt = 0; tt < QT; ++tt) {
                const int t = q * QT + tt;
                const float4 ka = *reinterpret_cast<const float4 *>(&Ks[x][16 * t + 4 * g]);
                const float4 qa = x == m0 ? *reinterpret_cast<const float4 *>(&Qrow[16 * t + 4 * g])
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
                Pq[q] = mfma_16x16x4(ka.x, S[t][0], Pq[q]);
                Zq[q] = mfma_16x16x4(qa.x, S[t][0], Zq[q]);
                Pq[q] = mfma_16x16x4(ka.y, S[t][1], Pq[q]);
                Zq[q] = mfma_16x16x4(qa.y, S[t][1], Zq[q]);
                Pq[q] = mfma_16x16x4(ka.z, S[t][2], Pq[q]);
                Zq[q] = mfma_16x16x4(qa.z, S[t][2], Zq[q]);
                Pq[q] = mfma_16x16x4(ka.w, S[t][3], Pq[q]);
                Zq[q] = mfma_16x16x4(qa.w, S[t][3], Zq[q]);
            }
        }
        f4 P, Z;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            P[c] = (Pq[0][c] + Pq[1][c]) + (Pq[2][c] + Pq[3][c]);
            Z[c] = (Zq[0][c] + Zq[1][c]) + (Zq[2][c] + Zq[3][c]);
        }
        f4 R, OC;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = 4 * g + c;
            const bool on = m >= m0 && m < m1;
            const float bb = on ? bt : 0.f;
            const float vb = bb * (on ? vv : 0.f);
            const float fresh = __builtin_fmaf(-(bb * gm[c]), P[c], vb);
            R[c] = on ? fresh : (m < m0 ? Rkeep[c] : 0.f);
            Rkeep[c] = on ? fresh : Rkeep[c];
            OC[c] = gm[c] * Z[c];
        }
        f4 U = f4_zero();
        U = mfma_16x16x4(trow.x, R[0], U);
        U = mfma_16x16x4(trow.y, R[1], U);
        U = mfma_16x16x4(trow.z, R[2], U);
        U = mfma_16x16x4(trow.w, R[3], U);
#pragma unroll
        for (int c = 0; c < 4; ++c) U[c] = U[c] + 0.f;
        f4 O = OC;
        O = mfma_16x16x4(brow.x, U[0], O);
        O = mfma_16x16x4(brow.y, U[1], O);
        O = mfma_16x16x4(brow.z, U[2], O);
        O = mfma_16x16x4(brow.w, U[3], O);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (4 * g + c == m0) IO::store1(p.out, (size_t)n * vrow + (size_t)h * p.dv + row0 + x, O[c] + 0.f);
        if (full) {
            const float w0 = dwv.x * U[0], w1 = dwv.y * U[1], w2 = dwv.z * U[2], w3 = dwv.w * U[3];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                f4 C = f4{g15 * S[t][0], g15 * S[t][1], g15 * S[t][2], g15 * S[t][3]};
                C = mfma_16x16x4(Ks[4 * g + 0][16 * t + x], w0, C);
                C = mfma_16x16x4(Ks[4 * g + 1][16 * t + x], w1, C);
                C = mfma_16x16x4(Ks[4 * g + 2][16 * t + x], w2, C);
                C = mfma_16x16x4(Ks[4 * g + 3][16 * t + x], w3, C);
                S[t] = C;
            }
        }
        // this tile's outgoing state (written in place only when the chunk closed) and R rows
        if (!inplace || full) {
            float *dst = p.out_S + (((size_t)n * p.hv + h) * p.dv + row0 + x) * DK;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                *reinterpret_cast<float4 *>(dst + 16 * t + 4 * g) = make_float4(S[t][0], S[t][1], S[t][2], S[t][3]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int m = 4 * g + c;
            if (m >= first && m < mo) p.out_r[(((size_t)n * kCk + m) * p.hv + h) * p.dv + row0 + x] = Rkeep[c];
        }
    }
    // the open chunk's decay factors, betas and keys, and the token count
    if (lane >= first && lane < mo) {
        const size_t e = ((size_t)n * kCk + lane) * p.hv + h;
        p.out_a[e] = decs[lane];
        p.out_b[e] = bets[lane];
    }
    if (h % G == 0) {
        for (int it = lane; it < kCk * (DK / 4); it += 64) {
            const int m = it / (DK / 4), c = 4 * (it % (DK / 4));
            if (m < first || m >= mo) continue;
            float4 kv;
            if (m >= (full ? 0 : m0))
                kv = IO::load4(p.k, ((size_t)(n - c0 + m) * p.hk + kh) * DK + c);
            else
                kv = *reinterpret_cast<const float4 *>(p.in_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + c);
            *reinterpret_cast<float4 *>(p.out_k + (((size_t)n * kCk + m) * p.hk + kh) * DK + c) = kv;
        }
        if (h == 0 && lane == 0) p.out_count[n] = mo;
    }
}

template <class IO, int DK, int MODE>
hipError_t chunked_launch(const ChunkedParams &p, hipStream_t s) {
    if (p.ws_slots > 0 && (MODE == 1 || p.cu_seqlens)) {  // (the decode kernel forms its own tables)
        const unsigned gx = p.cu_seqlens ? (unsigned)p.ws_slots : (unsigned)p.n_seqs;
        hipLaunchKernelGGL((gdn_chunk_prep_kernel<DK, IO, MODE == 1>), dim3(gx, (unsigned)p.hk), dim3(256), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (MODE != 1 && !p.cu_seqlens) {  // one token per sequence, no cu_seqlens
        hipLaunchKernelGGL((gdn_chunk_decode_kernel<DK, IO>), dim3((unsigned)((int64_t)p.n_seqs * p.hv)), dim3(64), 0,
                           s, p);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((int64_t)p.n_seqs * p.hv * (p.dv / 16)));
    switch (p.waves) {
        case 1: hipLaunchKernelGGL((gdn_chunk_main_kernel<DK, IO, 1, MODE>), grid, dim3(64), 0, s, p); break;
        case 2: hipLaunchKernelGGL((gdn_chunk_main_kernel<DK, IO, 2, MODE>), grid, dim3(128), 0, s, p); break;
        case 4: hipLaunchKernelGGL((gdn_chunk_main_kernel<DK, IO, 4, MODE>), grid, dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class IO, int MODE>
hipError_t chunked_io(const ChunkedParams &p, hipStream_t s) {
    switch (p.dk) {
        case 64: return chunked_launch<IO, 64, MODE>(p, s);
        case 128: return chunked_launch<IO, 128, MODE>(p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int MODE>
hipError_t chunked_mode(const ChunkedParams &p, int io_dtype, hipStream_t s) {
    return io_dtype == GDN_BF16 ? chunked_io<IoBf16, MODE>(p, s) : chunked_io<IoF32, MODE>(p, s);
}

}  // namespace

hipError_t launch_chunked(const ChunkedParams &p, int io_dtype, hipStream_t s) {
    return p.lean ? chunked_mode<2>(p, io_dtype, s) : chunked_mode<0>(p, io_dtype, s);
}

hipError_t launch_chunked_bwd_walk(const ChunkedParams &p, int io_dtype, hipStream_t s) {
    return chunked_mode<1>(p, io_dtype, s);
}

}  // namespace gdn
