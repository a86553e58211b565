// gdn_internal.hpp -- host-side plumbing shared by the C-ABI front end (gdn_api.hip)
// and the per-head-dim kernel translation units (gdn_dk*.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Largest batch whose sequences the prefill kernel orders longest first.
constexpr int kMaxRankedSeqs = 128;

// Snapshot spacing must be a multiple of this (and so of every token block, which
// bounds snapshots to one per block).
constexpr int kSnapshotGranule = 16;

// Kernel arguments of the varlen prefill (passed by value as the kernarg segment).
// Initial and final states are addressed by slot: slot n of h0 / hT for sequence n,
// or, when src_idx / dst_idx are given, slot src_idx[n] / dst_idx[n] of a pool of
// pool_size entries (a slot outside [0, pool_size) means none: zero state, or no
// write).  Snapshots (snap_block > 0) store the state reached at every absolute
// position that is a multiple of snap_block, counting pos0[n] tokens already
// behind sequence n, into pool slots snap_idx[n * snap_per_seq + j].
struct PrefillParams {
    const void *q, *k, *v;
    const float *g, *beta, *h0;
    const int32_t *cu_seqlens;
    void *out;
    float *hT;
    const int32_t *src_idx, *dst_idx;  // null: slot = sequence index
    const int32_t *pos0;               // null: no tokens behind any sequence
    const int32_t *snap_idx;           // [n_seqs][snap_per_seq]
    float *snap;                       // snapshot pool
    int64_t total_tokens;
    int32_t n_seqs, hk, hv, dv;
    int32_t pool_size;                 // slots of h0 / hT / snap when indexed
    int32_t snap_block, snap_per_seq;  // 0: no snapshots
    int32_t rank_by_length;  // workgroups take sequences longest first (n_seqs <= kMaxRankedSeqs)
    int32_t tiles;           // row tiles per value head (set by the launcher)
    // fused preprocessing (gdn_preproc): GDN_PRE_* flags; g / beta hold logits when gated
    const float *A_log, *dt_bias;
    float pre_eps;
    int32_t pre_flags;
    float *save_p;  // [T][hv][dv] p_t = S_{t-1} k_t for the backward, or null (extended instance only)
};

// Kernel arguments of one decode step.
struct DecodeParams {
    const void *q, *k, *v;
    const float *g, *beta;
    float *pool;
    const int32_t *state_idx;
    void *out;
    int32_t batch, hk, hv, dv, pool_size;
    const float *A_log, *dt_bias;  // fused preprocessing, as in PrefillParams
    float pre_eps;
    int32_t pre_flags;
};

// Kernel arguments of the short convolution (gdn_short_conv).
struct ConvParams {
    const void *x;
    const float *w, *bias;
    const int32_t *cu_seqlens, *src_idx, *dst_idx;
    void *state;
    void *y;
    int64_t total_tokens;
    int32_t n_seqs, channels, taps, pool_size, silu;
};
hipError_t launch_short_conv(const ConvParams &p, int io_dtype, hipStream_t s);

// Kernel arguments of the convolution's backward (gdn_short_conv_backward).
struct ConvBwdParams {
    const void *x;                    // io dtype [T][C]
    const float *w, *bias;            // [C][K], [C] or null
    const int32_t *cu_seqlens, *src_idx;
    const void *state;                // io dtype [P][C][K-1]: the states the forward read
    const float *dy;                  // [T][C]
    float *dx, *dw, *dbias, *dstate;  // [T][C], [C][K], [C] or null, [N][C][K-1] or null
    float *partial;                   // workspace: per token block and channel, K + 1 partial sums
    int64_t total_tokens;
    int32_t n_seqs, channels, taps, pool_size, silu;
};
uint64_t conv_bwd_workspace_bytes(int64_t T, int64_t C, int K);
hipError_t launch_short_conv_backward(const ConvBwdParams &p, int io_dtype, hipStream_t s);

// Kernel arguments of the backward (gdn_bwd_varlen).  The four row passes and the
// two finishing kernels share them; each reads and writes the parts it needs.
struct BwdParams {
    const void *q, *k, *v, *dout;    // io dtype
    const float *g, *beta, *h0, *dhT;
    const int32_t *cu_seqlens;
    float *grad_q, *grad_k, *grad_v, *grad_g, *grad_beta, *grad_h0;  // outputs (grad_h0 may be null)
    // workspace
    float *rbuf;   // [T][hv][dv]   r_t = v_t - a_t S_{t-1} k_t  (u_t = beta_t r_t)
    float *dubuf;  // [T][hv][dv]   du_t = dL/du_t
    float *dkbuf;  // [T][hv][dk]   dk of each value head
    float *dqbuf;  // [T][hv][dk]   dq of each value head
    float *cbuf;   // [T][hv]       q_t . dq_t - dv_t . v_t (the gate term)
    float *hT;     // [N][hv][dv][dk] final state (when dhT is given)
    const float *saved_p;  // [T][hv][dv] p_t saved by the training forward: F0 is skipped
    int64_t total_tokens;
    int32_t n_seqs, hk, hv, dk, dv;
    int32_t rank_by_length;
};
hipError_t launch_backward(const BwdParams &p, int io_dtype, hipStream_t s);
// Workspace layout of the backward: byte offsets of rbuf, dubuf, dkbuf, dqbuf,
// cbuf and hT, and the total.
struct BwdWorkspace {
    uint64_t p, du, dk, dq, c, hT, total;
};
BwdWorkspace backward_workspace(int64_t T, int64_t N, int hv, int dk, int dv);

// Kernel arguments of the chunked form with its replaying decode (gdn_fwd_chunked).
// A chunked state is the state at the start of the open chunk plus that chunk's
// keys, R rows beta (v - Gam S0 k), decay factors a and betas, and its token count.
constexpr int kChunkLen = 16;
struct ChunkedParams {
    const void *q, *k, *v;
    const float *g, *beta;
    const int32_t *cu_seqlens;
    const float *in_S, *in_k, *in_r, *in_a, *in_b;  // null in_S: zero state; null in_count: empty chunk
    const int32_t *in_count;
    float *out_S, *out_k, *out_r, *out_a, *out_b;
    int32_t *out_count;
    void *out;
    float *ws;         // per (workspace slot, value head) records of kChunkRec floats
    int64_t ws_slots;  // slots in the workspace
    int64_t total_tokens;
    int32_t n_seqs, hk, hv, dk, dv;
    int32_t rank_by_length;  // workgroups take sequences longest first (n_seqs <= kMaxRankedSeqs)
    int32_t inplace;         // out shares S, k, r, a and b with in (one-token calls only)
    int32_t waves;           // waves per 16-row tile: 1, 2 or 4 (each owns 4 / waves dk quarters)
    int32_t lean;            // the lean form of the main kernel (few tokens per sequence; same bits)
    // Forward walk of the chunked backward (launch_chunked_bwd_walk): records of
    // kChunkRecBwd floats, no outputs or outgoing chunked state; instead the state at
    // every chunk's start (ck: [slot][hv][dv][dk], like a state), x = v - Gam P of every
    // token ([T][hv][dv]) and the partial sums of <dhT, hT> ([N][hv][dv / 16][4 dk quarters]).
    float *ck;
    float *xv;
    const float *dhT;
    float *hdot;
};
hipError_t launch_chunked(const ChunkedParams &p, int io_dtype, hipStream_t s);
hipError_t launch_chunked_bwd_walk(const ChunkedParams &p, int io_dtype, hipStream_t s);

// The fused preprocessing as a pass of its own and its gradients (gdn_preproc.hip).
struct PreParams {
    const void *q, *k;                            // raw queries and keys, io dtype [T][hk][dk]
    const float *a, *b;                           // gate and beta logits (or g, beta) [T][hv]
    float *qn, *kn, *g, *beta;                    // forward: the preprocessed values (fp32)
    const float *dqn, *dkn, *dg, *dbeta;          // backward: their gradients (fp32)
    float *dq, *dk, *da, *db, *dA_log, *ddt_bias; // backward: the raw inputs' gradients
    const float *A_log, *dt_bias;
    float eps;
    int32_t flags;
    int64_t total_tokens;
    int32_t hk, hv;
};
hipError_t launch_preprocess(const PreParams &p, int dk, int io_dtype, bool backward, hipStream_t s);

// Kernel arguments of the reverse walk of the chunked backward (gdn_bwd_chunked).
struct BwdChunkParams {
    const void *q, *k, *v, *dout;     // io dtype
    const float *beta, *dhT;
    const int32_t *cu_seqlens;
    const float *rec, *ck, *xv, *hdot;  // from the prep kernel and the forward walk
    float *grad_v, *grad_g, *grad_beta, *grad_h0;
    float *dqh, *dkh;                 // [parts][T][hv][dk]: dq, dk of each value head and part
                                      // (the outputs when hv == hk and parts == 1)
    float *dbeta_part, *dg_part;      // [parts][T][hv] (parts > 1)
    float *grad_q, *grad_k;           // [T][hk][dk]
    int64_t ws_slots, total_tokens;
    int32_t n_seqs, hk, hv, dk, dv;
    int32_t rank_by_length;
    int32_t hdot_parts;               // partial sums of <dhT, hT> per (sequence, value head)
    int32_t parts;                    // workgroups per (sequence, value head), each a share of the rows
    int32_t plain;                    // no wave specialization (same bits; for comparison)
};
hipError_t launch_bwd_chunked(const BwdChunkParams &p, int io_dtype, hipStream_t s);


// Workspace of the chunked form: one record per (chunk a call touches, value head).
// Sequence n's chunks take slots chunk_slot_base(cu[n], n) + j: floor(cu[n] / 16)
// + 2 n grows by at least floor(len / 16) + 2 from one sequence to the next, which
// covers the at most ceil((15 + len) / 16) chunks a sequence of len tokens touches,
// so floor(T / 16) + 2 N + 2 slots hold every call.
constexpr int kChunkRec = 576;  // floats: T[16][16], B[16][16], Gam[16], D[16], a[16], beta[16]
constexpr int kRecT = 0, kRecB = 256, kRecGam = 512, kRecD = 528, kRecDecay = 544, kRecBeta = 560;
// The backward's record adds Gam_{m,s} (s <= m) and Gam_{m,s} (k_m . k_s) (s < m), zero elsewhere.
constexpr int kChunkRecBwd = 1088;
constexpr int kRecGm = 576, kRecAb = 832;
__host__ __device__ inline int64_t chunk_slot_base(int64_t cu_n, int n) { return cu_n / kChunkLen + 2 * (int64_t)n; }
__host__ __device__ inline int64_t chunk_ws_slots(int64_t T, int64_t N) { return T / kChunkLen + 2 * N + 2; }

// A launch shape: `lanes` lanes hold one state row, each lane holds `rows` rows,
// and a workgroup has `waves` waves; it owns waves * (64 / lanes) * rows
// consecutive rows of one value head.
struct Plan {
    int lanes;
    int rows;
    int waves;
};

// Per-head-dim entry points, defined in gdn_dk{16,32,64,128}.hip.
#define GDN_DECLARE_DK(DK)                                                                     \
    bool plan_available_dk##DK(bool decode, int io_dtype, Plan plan);                                     \
    hipError_t launch_prefill_dk##DK(const PrefillParams &p, int io_dtype, Plan plan, hipStream_t s); \
    hipError_t launch_decode_dk##DK(const DecodeParams &p, int io_dtype, Plan plan, hipStream_t s);
GDN_DECLARE_DK(16)
GDN_DECLARE_DK(32)
GDN_DECLARE_DK(64)
GDN_DECLARE_DK(128)
#undef GDN_DECLARE_DK

}  // namespace gdn
