// gdn_bwd.hip -- gradients of the recurrent forward (gdn_bwd_varlen).
//
// Forward step of token t (per sequence and value head; S is dv x dk, row j):
//     p_t = S_{t-1} k_t,   u_t = beta_t (v_t - a_t p_t),   S_t = a_t S_{t-1} + u_t k_t^T,
//     o_t = S_t q_t,       a_t = exp(g_t)
// (the gated delta rule of Yang, Kautz and Hatamizadeh, ICLR 2025; the page "Defending
// Against the Training-Inference Numeric Mismatch in RL (Especially Linear
// Attention)", section 3.2, runs it token by token in every forward and keeps the
// training backward as a separate kernel).
//
// With D_t = dL/dS_t, the adjoint walked from the last token back is
//     D  <- D + dO_t q_t^T;   du_t = D k_t;   D <- a_t (D - beta_t du_t k_t^T)
// and the gradients are
//     dv_t = beta_t du_t,  dbeta_t = du_t . (v_t - a_t p_t),
//     dq_t = S_t^T dO_t,   dk_t = D_t^T u_t + S_{t-1}^T (-a_t beta_t du_t),
//     dg_t = <dhT, hT> + sum_{s >= t} (dO_s . o_s - dv_s . v_s),   dh0 = D_0.
// The gate gradient needs no state inner product: with Phi_t = <D_t, S_t>,
// Phi_{t-1} = dO_{t-1} . o_{t-1} + dg_t and Phi_t = dg_t + beta_t du_t . v_t, so dg is a
// reverse running sum within the sequence; dO_s . o_s = q_s . dq_s.
//
// Every gradient is then a row-wise quantity of some state, which keeps the
// forward's layout (L lanes hold one state row, row dots finished by DPP, no
// reduction across rows) in each of four passes over the tokens:
//
//   F0 forward  over S   (rows j, columns i): r_t = v_t - a_t p_t, and hT
//   R1 reverse  over D   (rows j, columns i): du_t, and dh0 = D_0
//   R2 reverse  over D^T (rows i, columns j): (D_t^T u_t)_i             -> dk
//   F3 forward  over S^T (rows i, columns j): (S_{t-1}^T w_t)_i, w_t = -a_t beta_t du_t,
//                                            and (S_t^T dO_t)_i          -> dk, dq
//
// then one kernel per (token, key head) sums the value heads of a key head, forms
// dv, dbeta and the gate term, and one per (sequence, value head) runs the reverse
// sum for dg.  Every sum has a fixed order and nothing crosses sequences, so the
// gradients are deterministic and do not depend on the batch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.hpp"
#include "gdn_kernels.hpp"

#pragma clang fp contract(off)

namespace gdn {
namespace {

enum BwdPass { kF0 = 0, kR1 = 1, kR2 = 2, kF3 = 3 };

constexpr int kBwdLanes = 8;   // lanes per state row
constexpr int kBwdWaves = 4;   // waves per workgroup
constexpr int kBwdRows = kBwdWaves * (64 / kBwdLanes);  // rows per workgroup (32)
constexpr int kBwdThreads = kBwdWaves * 64;
constexpr int kBwdTB = 16;     // tokens per staged block

template <int C>
__device__ __forceinline__ float lane_dot(const float (&x)[C], const float (&y)[C]) {
    constexpr int K = C >= 16 ? 4 : (C >= 8 ? 2 : 1);  // independent chains
    float acc[K];
#pragma unroll
    for (int c = 0; c < K; ++c) acc[c] = x[c] * y[c];
#pragma unroll
    for (int c = K; c < C; ++c) acc[c % K] = __builtin_fmaf(x[c], y[c], acc[c % K]);
    if constexpr (K == 1) return acc[0];
    else if constexpr (K == 2) return acc[0] + acc[1];
    else return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// LDS position (in 4-float chunks) of lane lam's j-th chunk of a staged column vector.
// The 8 lanes of a row read their j-th chunks together; with 16 columns per lane
// (NC = 128) chunk j of lanes lam and lam + 4 would fall on the same banks, so those
// lanes take their chunks in a rotated order.  Narrower rows do not conflict.
template <int NC>
__device__ __forceinline__ int bwd_chunk_slot(int lam, int j) {
    constexpr int CH = NC / kBwdLanes / 4;  // chunks per lane
    if constexpr (CH == 4) return lam * CH + ((j + (lam >> 2)) & 3);
    else return lam * CH + j;
}

template <int NC>
struct alignas(16) BwdLds {
    float cv[3][kBwdTB][NC];        // column vectors of each staged token (up to three)
    float rs[2][kBwdTB][kBwdRows];  // row scalars of this tile (up to two)
    float a[kBwdTB], b[kBwdTB];  // exp(g), beta
};

// One workgroup = (sequence, value head, tile of 32 state rows) for pass PASS.
// NC: length of a state row (dk for F0 / R1, dv for R2 / F3).
template <int PASS, int NC, class IO>
__global__ __launch_bounds__(kBwdThreads) void gdn_bwd_pass_kernel(BwdParams p) {
    constexpr int C = NC / kBwdLanes;
    constexpr bool REV = (PASS == kR1 || PASS == kR2);
    __shared__ BwdLds<NC> Ld;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lam = lane % kBwdLanes, grp = lane / kBwdLanes;
    const int rows = (PASS == kF0 || PASS == kR1) ? p.dv : p.dk;  // state rows of this pass
    const int tiles = rows / kBwdRows;
    const int tile = blockIdx.x % tiles;
    const int h = (blockIdx.x / tiles) % p.hv;
    const int rank = blockIdx.x / (tiles * p.hv);
    const int n = p.rank_by_length ? seq_by_length_rank(p.cu_seqlens, p.n_seqs, rank, tid, kBwdThreads) : rank;
    const int kh = h / (p.hv / p.hk);
    const int lrow = wave * (64 / kBwdLanes) + grp;  // row within the tile
    const int row = tile * kBwdRows + lrow;
    const int col0 = lam * C;
    int lchunk[C / 4];  // LDS float offsets of this lane's column chunks
#pragma unroll
    for (int j = 0; j < C / 4; ++j) lchunk[j] = 4 * bwd_chunk_slot<NC>(lam, j);

    int64_t tb = p.cu_seqlens[n], te = p.cu_seqlens[n + 1];
    tb = tb < 0 ? 0 : (tb > p.total_tokens ? p.total_tokens : tb);
    te = te < tb ? tb : (te > p.total_tokens ? p.total_tokens : te);

    // state slice: row `row`, columns col0 .. col0 + C - 1
    const size_t sbase = ((size_t)n * p.hv + h) * (size_t)p.dv * p.dk;
    float X[C];
    {
        const float *init = (PASS == kF0 || PASS == kF3) ? p.h0 : p.dhT;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            float x = 0.f;
            if (init) {
                // F0 / R1 hold rows j (dv) of a dv x dk matrix; R2 / F3 hold its transpose
                x = (PASS == kF0 || PASS == kR1) ? init[sbase + (size_t)row * p.dk + col0 + c]
                                                 : init[sbase + (size_t)(col0 + c) * p.dk + row];
            }
            X[c] = x;
        }
    }

    const int64_t len = te - tb;
    const int nblk = (int)((len + kBwdTB - 1) / kBwdTB);
    // Forward passes take block blk from the start, reverse passes from the end;
    // slot ti of a block is token s0 + ti.
    auto block_first = [&](int blk) -> int64_t {
        const int64_t t0 = REV ? (te - (int64_t)(blk + 1) * kBwdTB) : (tb + (int64_t)blk * kBwdTB);
        return t0 < tb ? tb : t0;
    };
    auto block_len = [&](int blk) -> int {
        const int64_t t0 = REV ? (te - (int64_t)(blk + 1) * kBwdTB) : (tb + (int64_t)blk * kBwdTB);
        const int64_t s1 = (t0 + kBwdTB > te) ? te : t0 + kBwdTB;
        return (int)(s1 - (t0 < tb ? tb : t0));
    };

    // Staging: a block's global reads go to registers, then to LDS.  (Issuing them
    // one block ahead measured no faster: the other waves on the SIMD already
    // cover their latency, and the registers held across a block cost occupancy.)
    // Column items are four columns of one token; row items one row of one token.
    constexpr int NC4 = NC / 4;
    constexpr int CITEMS = (kBwdTB * NC4 + kBwdThreads - 1) / kBwdThreads;
    constexpr int RITEMS = (kBwdTB * kBwdRows + kBwdThreads - 1) / kBwdThreads;
    float4 cr[CITEMS][3];
    float rr[RITEMS][2];
    float sa = 0.f, sb = 0.f;
    auto fetch = [&](int blk) {
        const int64_t s0 = block_first(blk);
        const int nt = block_len(blk);
#pragma unroll
        for (int it = 0; it < CITEMS; ++it) {
            const int idx = tid + it * kBwdThreads;
            if (idx >= nt * NC4) continue;
            const int ti = idx / NC4, c = 4 * (idx % NC4);
            const int64_t t = s0 + ti;
            if constexpr (PASS == kF0 || PASS == kR1) {
                const size_t qk = ((size_t)t * p.hk + kh) * p.dk + c;
                if constexpr (PASS == kF0) {
                    cr[it][0] = IO::load4(p.k, qk);
                } else {
                    cr[it][0] = IO::load4(p.q, qk);
                    cr[it][1] = IO::load4(p.k, qk);
                }
            } else {
                const size_t vv = ((size_t)t * p.hv + h) * p.dv + c;
                const float b = p.beta[(size_t)t * p.hv + h];
                const float4 r = *reinterpret_cast<const float4 *>(p.rbuf + vv);
                const float4 du = *reinterpret_cast<const float4 *>(p.dubuf + vv);
                const float4 u = make_float4(b * r.x, b * r.y, b * r.z, b * r.w);
                const float4 dvv = make_float4(b * du.x, b * du.y, b * du.z, b * du.w);
                const float4 dO = IO::load4(p.dout, vv);
                if constexpr (PASS == kR2) {
                    cr[it][0] = dO;
                    cr[it][1] = u;
                    cr[it][2] = dvv;
                } else {
                    const float na = -decay_factor(p.g[(size_t)t * p.hv + h]);  // w_t = -a_t beta_t du_t
                    cr[it][0] = make_float4(na * dvv.x, na * dvv.y, na * dvv.z, na * dvv.w);
                    cr[it][1] = u;
                    cr[it][2] = dO;
                }
            }
        }
#pragma unroll
        for (int it = 0; it < RITEMS; ++it) {
            const int idx = tid + it * kBwdThreads;
            if (idx >= nt * kBwdRows) continue;
            const int ti = idx / kBwdRows, r = idx % kBwdRows;
            const int64_t t = s0 + ti;
            const int rw = tile * kBwdRows + r;
            if constexpr (PASS == kF0) {
                rr[it][0] = IO::load1(p.v, ((size_t)t * p.hv + h) * p.dv + rw);
            } else if constexpr (PASS == kR1) {
                rr[it][0] = IO::load1(p.dout, ((size_t)t * p.hv + h) * p.dv + rw);
            } else if constexpr (PASS == kR2) {
                const size_t qk = ((size_t)t * p.hk + kh) * p.dk + rw;
                rr[it][0] = IO::load1(p.q, qk);
                rr[it][1] = IO::load1(p.k, qk);
            } else {
                rr[it][0] = IO::load1(p.k, ((size_t)t * p.hk + kh) * p.dk + rw);
                rr[it][1] = p.dkbuf[((size_t)t * p.hv + h) * p.dk + rw];  // R2's term of dk
            }
        }
        if (tid < nt) {
            const int64_t t = s0 + tid;
            sa = decay_factor(p.g[(size_t)t * p.hv + h]);
            sb = p.beta[(size_t)t * p.hv + h];
        }
    };
    auto commit = [&](int blk) {
        const int nt = block_len(blk);
        constexpr int NV = (PASS == kF0) ? 1 : (PASS == kR1 ? 2 : 3);
        constexpr int NR = (PASS == kR2 || PASS == kF3) ? 2 : 1;
#pragma unroll
        for (int it = 0; it < CITEMS; ++it) {
            const int idx = tid + it * kBwdThreads;
            if (idx >= nt * NC4) continue;
            const int ch = idx % NC4, ti = idx / NC4;
            const int slot = bwd_chunk_slot<NC>(ch / (C / 4), ch % (C / 4));
#pragma unroll
            for (int v = 0; v < NV; ++v) *reinterpret_cast<float4 *>(&Ld.cv[v][ti][4 * slot]) = cr[it][v];
        }
#pragma unroll
        for (int it = 0; it < RITEMS; ++it) {
            const int idx = tid + it * kBwdThreads;
            if (idx >= nt * kBwdRows) continue;
            const int ti = idx / kBwdRows, r = idx % kBwdRows;
#pragma unroll
            for (int v = 0; v < NR; ++v) Ld.rs[v][ti][r] = rr[it][v];
        }
        if (tid < nt) {
            Ld.a[tid] = sa;
            Ld.b[tid] = sb;
        }
    };

    for (int blk = 0; blk < nblk; ++blk) {
        const int64_t s0 = block_first(blk);
        const int nt = block_len(blk);
        fetch(blk);
        commit(blk);
        __syncthreads();

        // ---- walk the block's tokens in this pass's direction
        // A token's LDS values go to one of two register sets, so the next token's
        // reads can be issued while this one computes.  Each row's results are kept
        // for 8 tokens (lane lam holds the token of step 8m + lam) and stored together.
        constexpr int NV = (PASS == kF0) ? 1 : (PASS == kR1 ? 2 : 3);
        constexpr int NR = (PASS == kR2 || PASS == kF3) ? 2 : 1;
        struct Tok {
            float v[NV][C];
            float r[NR];
            float a, b;
        };
        auto slot_of = [&](int stp) { return REV ? nt - 1 - stp : stp; };
        auto load_tok = [&](Tok &X_, int stp) {
            const int ti = slot_of(stp);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int j = 0; j < C / 4; ++j) {
                    const float4 x = *reinterpret_cast<const float4 *>(&Ld.cv[v][ti][lchunk[j]]);
                    X_.v[v][4 * j] = x.x; X_.v[v][4 * j + 1] = x.y; X_.v[v][4 * j + 2] = x.z; X_.v[v][4 * j + 3] = x.w;
                }
#pragma unroll
            for (int v = 0; v < NR; ++v) X_.r[v] = Ld.rs[v][ti][lrow];
            X_.a = Ld.a[ti];
            X_.b = Ld.b[ti];
        };
        float ob0 = 0.f, ob1 = 0.f;  // kept results (F3 keeps two)
        // row output of token slot ti: rbuf / dubuf (rows dv) or dkbuf / dqbuf (rows dk)
        auto out_index = [&](int ti) -> size_t {
            return ((size_t)(s0 + ti) * p.hv + h) * (size_t)((PASS == kF0 || PASS == kR1) ? p.dv : p.dk) + row;
        };
        auto flush = [&](int stp) {  // after step stp: store the kept results of steps (stp & ~7) .. stp
            const int sl = (stp & ~7) + lam;
            if (sl > stp) return;
            const size_t o = out_index(slot_of(sl));
            if constexpr (PASS == kF0) p.rbuf[o] = ob0;
            else if constexpr (PASS == kR1) p.dubuf[o] = ob0;
            else if constexpr (PASS == kR2) p.dkbuf[o] = ob0;
            else {
                p.dkbuf[o] = ob0;
                p.dqbuf[o] = ob1;
            }
        };
        auto compute = [&](const Tok &T_, int stp) {
            const float a = T_.a, b = T_.b;
            float y0 = 0.f, y1 = 0.f;
            if constexpr (PASS == kF0) {
                // p = S_{t-1} k;  r = v - a p;  S = a S + (beta r) k^T
                const float pt = lane_sum<kBwdLanes>(lane_dot<C>(X, T_.v[0]));
                y0 = T_.r[0] - a * pt;
                const float u = b * y0;
#pragma unroll
                for (int c = 0; c < C; ++c) X[c] = __builtin_fmaf(a, X[c], u * T_.v[0][c]);
            } else if constexpr (PASS == kR1) {
                // D += dO q^T;  du = D k;  D = a (D - beta du k^T)
#pragma unroll
                for (int c = 0; c < C; ++c) X[c] = __builtin_fmaf(T_.r[0], T_.v[0][c], X[c]);
                y0 = lane_sum<kBwdLanes>(lane_dot<C>(X, T_.v[1]));
                const float bdu = b * y0;
#pragma unroll
                for (int c = 0; c < C; ++c) X[c] = a * __builtin_fmaf(-bdu, T_.v[1][c], X[c]);
            } else if constexpr (PASS == kR2) {
                // E = D^T:  E += q dO^T;  y = E u;  E = a (E - k dv^T)
#pragma unroll
                for (int c = 0; c < C; ++c) X[c] = __builtin_fmaf(T_.r[0], T_.v[0][c], X[c]);
                y0 = lane_sum<kBwdLanes>(lane_dot<C>(X, T_.v[1]));
#pragma unroll
                for (int c = 0; c < C; ++c) X[c] = a * __builtin_fmaf(-T_.r[1], T_.v[2][c], X[c]);
            } else {
                // P = S^T:  y1 = P w (old state);  P = a P + k u^T;  y2 = P dO (new state)
                y0 = T_.r[1] + lane_sum<kBwdLanes>(lane_dot<C>(X, T_.v[0]));  // plus R2's term of dk
#pragma unroll
                for (int c = 0; c < C; ++c) X[c] = __builtin_fmaf(a, X[c], T_.r[0] * T_.v[1][c]);
                y1 = lane_sum<kBwdLanes>(lane_dot<C>(X, T_.v[2]));
            }
            if (lam == (stp & 7)) {
                ob0 = y0;
                ob1 = y1;
            }
        };
        if (nt == kBwdTB && (PASS == kF0 || PASS == kR1)) {
            // F0 and R1 carry their dot on the recurrence's critical path, so the next
            // token's reads go ahead of it.  (R2 and F3 would need more than 168
            // registers for a second set and lose a wave per SIMD: measured slower.)
            Tok A, B;
            load_tok(A, 0);
#pragma unroll
            for (int stp = 0; stp < kBwdTB; stp += 2) {
                load_tok(B, stp + 1);
                compute(A, stp);
                if (stp + 2 < kBwdTB) load_tok(A, stp + 2);
                compute(B, stp + 1);
                if ((stp + 1) % 8 == 7) flush(stp + 1);
            }
        } else if (nt == kBwdTB) {
#pragma unroll
            for (int stp = 0; stp < kBwdTB; ++stp) {
                Tok A;
                load_tok(A, stp);
                compute(A, stp);
                if ((stp & 7) == 7) flush(stp);
            }
        } else {
            for (int stp = 0; stp < nt; ++stp) {
                Tok A;
                load_tok(A, stp);
                compute(A, stp);
                if ((stp & 7) == 7 || stp == nt - 1) flush(stp);
            }
        }
        __syncthreads();
    }

    // final states: hT after F0 (only needed for <dhT, hT>), dh0 = D_0 after R1
    float *dst = (PASS == kF0) ? (p.dhT ? p.hT : nullptr) : (PASS == kR1 ? p.grad_h0 : nullptr);
    if (dst) {
#pragma unroll
        for (int c = 0; c < C; c += 4)
            *reinterpret_cast<float4 *>(dst + sbase + (size_t)row * p.dk + col0 + c) =
                make_float4(X[c], X[c + 1], X[c + 2], X[c + 3]);
    }
}

// Sum over the 64 lanes of a wave (pairwise over lane index; every lane gets it).
__device__ __forceinline__ float wave_sum(float x) {
    x = group_sum<32>(x);
    return x + __shfl_xor(x, 32);
}

// One wave per (token, key head): dq and dk of the key head (its value heads in
// order), and per value head dv = beta du, dbeta = du . (v - a p) and the gate term
// c = q . dq_h - dv . v.
template <class IO>
__global__ __launch_bounds__(256) void gdn_bwd_finish_kernel(BwdParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= p.total_tokens * p.hk) return;
    const int64_t t = item / p.hk;
    const int kh = (int)(item % p.hk);
    const int G = p.hv / p.hk;
    for (int i = lane; i < p.dk; i += 64) {
        float sq = 0.f, sk = 0.f;
        for (int m = 0; m < G; ++m) {
            const size_t o = ((size_t)t * p.hv + kh * G + m) * p.dk + i;
            sq += p.dqbuf[o];
            sk += p.dkbuf[o];
        }
        const size_t oq = ((size_t)t * p.hk + kh) * p.dk + i;
        p.grad_q[oq] = sq;
        p.grad_k[oq] = sk;
    }
    for (int m = 0; m < G; ++m) {
        const int h = kh * G + m;
        const float b = p.beta[(size_t)t * p.hv + h];
        float db = 0.f, dvv = 0.f, qdq = 0.f;
        for (int j = lane; j < p.dv; j += 64) {
            const size_t o = ((size_t)t * p.hv + h) * p.dv + j;
            const float du = p.dubuf[o], v = IO::load1(p.v, o);
            const float dv = b * du;
            p.grad_v[o] = dv;
            db = __builtin_fmaf(du, p.rbuf[o], db);
            dvv = __builtin_fmaf(dv, v, dvv);
        }
        for (int i = lane; i < p.dk; i += 64)
            qdq = __builtin_fmaf(IO::load1(p.q, ((size_t)t * p.hk + kh) * p.dk + i),
                                 p.dqbuf[((size_t)t * p.hv + h) * p.dk + i], qdq);
        db = wave_sum(db);
        dvv = wave_sum(dvv);
        qdq = wave_sum(qdq);
        if (lane == 0) {
            p.grad_beta[(size_t)t * p.hv + h] = db;
            p.cbuf[(size_t)t * p.hv + h] = qdq - dvv;
        }
    }
}

// One workgroup per (sequence, value head): dg_t = <dhT, hT> + sum_{s >= t} c_s,
// accumulated in fp64.  Thread k owns a contiguous stretch of the sequence; the
// stretch sums are combined in a fixed order.
__global__ __launch_bounds__(256) void gdn_bwd_gate_kernel(BwdParams p) {
    __shared__ double red[256];
    const int tid = threadIdx.x;
    const int n = blockIdx.x / p.hv, h = blockIdx.x % p.hv;
    int64_t tb = p.cu_seqlens[n], te = p.cu_seqlens[n + 1];
    tb = tb < 0 ? 0 : (tb > p.total_tokens ? p.total_tokens : tb);
    te = te < tb ? tb : (te > p.total_tokens ? p.total_tokens : te);

    double base = 0.0;
    if (p.dhT) {  // <dhT, hT>
        const size_t s = ((size_t)n * p.hv + h) * (size_t)p.dv * p.dk;
        double acc = 0.0;
        for (int64_t e = tid; e < (int64_t)p.dv * p.dk; e += 256)
            acc += (double)p.dhT[s + e] * (double)p.hT[s + e];
        red[tid] = acc;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if (tid < w) red[tid] += red[tid + w];
            __syncthreads();
        }
        base = red[0];
        __syncthreads();
    }
    const int64_t len = te - tb;
    const int64_t per = (len + 255) / 256;
    const int64_t c0 = tb + tid * per, c1 = (c0 + per < te) ? c0 + per : te;
    double mine = 0.0;
    for (int64_t t = c0; t < c1; ++t) mine += (double)p.cbuf[(size_t)t * p.hv + h];
    red[tid] = mine;
    __syncthreads();
    // suffix over the stretches after this one, added in stretch order
    double after = base;
    for (int k = 255; k > tid; --k) after += red[k];
    double run = after;
    for (int64_t t = c1 - 1; t >= c0; --t) {
        run += (double)p.cbuf[(size_t)t * p.hv + h];
        p.grad_g[(size_t)t * p.hv + h] = (float)run;
    }
}

template <int PASS, int NC, class IO>
hipError_t launch_pass(const BwdParams &p, hipStream_t s) {
    const int rows = (PASS == kF0 || PASS == kR1) ? p.dv : p.dk;
    const dim3 grid((unsigned)((int64_t)p.n_seqs * p.hv * (rows / kBwdRows)));
    hipLaunchKernelGGL((gdn_bwd_pass_kernel<PASS, NC, IO>), grid, dim3(kBwdThreads), 0, s, p);
    return hipGetLastError();
}

template <int PASS, class IO>
hipError_t pass_for_dims(const BwdParams &p, hipStream_t s) {
    const int nc = (PASS == kF0 || PASS == kR1) ? p.dk : p.dv;
    switch (nc) {
        case 32: return launch_pass<PASS, 32, IO>(p, s);
        case 64: return launch_pass<PASS, 64, IO>(p, s);
        case 128: return launch_pass<PASS, 128, IO>(p, s);
        default: return hipErrorInvalidValue;
    }
}

// With p_t saved by the training forward, r = v - a p is formed elementwise in place
// of the F0 pass (same formula as F0's, on the forward's p).
template <class IO>
__global__ __launch_bounds__(256) void gdn_bwd_r_from_p_kernel(BwdParams p) {
    const int64_t n4 = p.total_tokens * p.hv * (p.dv / 4);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const int64_t e = 4 * i;
        const int64_t th = e / p.dv;  // token * hv + head
        const float a = decay_factor(p.g[th]);
        const float4 v = IO::load4(p.v, (size_t)e);
        const float4 pv = *reinterpret_cast<const float4 *>(p.saved_p + e);
        *reinterpret_cast<float4 *>(p.rbuf + e) = make_float4(v.x - a * pv.x, v.y - a * pv.y, v.z - a * pv.z, v.w - a * pv.w);
    }
}

template <class IO>
hipError_t backward_io(const BwdParams &p, hipStream_t s) {
    hipError_t e;
    if (p.saved_p) {
        const int64_t n4 = p.total_tokens * p.hv * (p.dv / 4);
        if (n4 > 0) {
            const int64_t blocks = (n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192;
            hipLaunchKernelGGL((gdn_bwd_r_from_p_kernel<IO>), dim3((unsigned)blocks), dim3(256), 0, s, p);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else if ((e = pass_for_dims<kF0, IO>(p, s)) != hipSuccess) {
        return e;
    }
    if ((e = pass_for_dims<kR1, IO>(p, s)) != hipSuccess) return e;
    if ((e = pass_for_dims<kR2, IO>(p, s)) != hipSuccess) return e;
    if ((e = pass_for_dims<kF3, IO>(p, s)) != hipSuccess) return e;
    if (p.total_tokens > 0) {
        const int64_t items = p.total_tokens * p.hk;
        hipLaunchKernelGGL((gdn_bwd_finish_kernel<IO>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(gdn_bwd_gate_kernel, dim3((unsigned)((int64_t)p.n_seqs * p.hv)), dim3(256), 0, s, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

uint64_t round_up(uint64_t x) { return (x + 255) & ~uint64_t(255); }

}  // namespace

BwdWorkspace backward_workspace(int64_t T, int64_t N, int hv, int dk, int dv) {
    BwdWorkspace w{};
    uint64_t off = 0;
    w.p = off;  off += round_up((uint64_t)T * hv * dv * 4);
    w.du = off; off += round_up((uint64_t)T * hv * dv * 4);
    w.dk = off; off += round_up((uint64_t)T * hv * dk * 4);
    w.dq = off; off += round_up((uint64_t)T * hv * dk * 4);
    w.c = off;  off += round_up((uint64_t)T * hv * 4);
    w.hT = off; off += round_up((uint64_t)N * hv * dv * dk * 4);
    w.total = off;
    return w;
}

hipError_t launch_backward(const BwdParams &p, int io_dtype, hipStream_t s) {
    return io_dtype == GDN_BF16 ? backward_io<IoBf16>(p, s) : backward_io<IoF32>(p, s);
}

}  // namespace gdn
