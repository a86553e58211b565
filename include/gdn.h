/*
 * gdn.h -- C ABI of the MI355X (gfx950) batch-invariant Gated DeltaNet recurrent forward.
 *
 * The operation.  For every sequence n and every value head h (key head
 * kh = h / (hv / hk)) the library walks the sequence's tokens in order against
 * that sequence's own fp32 state S (a dv x dk matrix, element S[j][i]):
 *
 *     a_t = exp(g_t)
 *     S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * which is the gated delta rule (Yang, Kautz, Hatamizadeh, "Gated Delta
 * Networks: Improving Mamba2 with Delta Rule", ICLR 2025).  Running this
 * token-by-token recurrence for prefill, for decode and for a trainer's
 * recompute alike, with one sequence's state touched by nothing but that
 * sequence's tokens and no reduction across sequences, is what the page
 * "Defending Against the Training-Inference Numeric Mismatch in RL (Especially
 * Linear Attention)" (section 3.2, operator level) relies on to make the forward
 * batch invariant.  No 1/sqrt(dk) scale is applied to q.
 *
 * Bitwise contract.  Every output element and every state element is produced
 * by a fixed sequence of fp32 operations that depends only on that sequence's
 * own inputs: never on the batch size, the position of the sequence in the
 * batch, the other sequences, the launch shape, or whether a token arrives by
 * gdn_fwd_varlen or by gdn_decode_step.  Splitting a sequence into several
 * calls and passing hT of one call as h0 of the next gives the same bits as one
 * call (the state is carried in fp32 without rounding).
 *
 * Layouts (all row-major, contiguous, token-major; T = total tokens):
 *     q, k        [T][hk][dk]     io dtype
 *     v, out      [T][hv][dv]     io dtype
 *     g, beta     [T][hv]         fp32 (g is the log of the decay, beta the write strength)
 *     h0, hT      [N][hv][dv][dk] fp32
 *     state pool  [P][hv][dv][dk] fp32 (decode, pooled prefill)
 *     cu_seqlens  [N+1]           int32, device memory
 *     state_idx   [B]             int32, device memory
 * All array pointers are device pointers (hipMalloc'd or equivalent), aligned to
 * 16 bytes.  The caller owns every buffer; the library allocates nothing, keeps
 * no pointer after a call returns and has no global state, so it is reentrant.
 * (The one exception is gdn_bwd_varlen_noalloc, which uses a fixed scratch array
 * that each device holds for the life of the process; see there.)
 * Work is enqueued on `stream` (a hipStream_t; NULL means the null stream) and
 * the call returns without synchronising the host.
 *
 * Errors.  Argument problems that the host can see are reported before anything
 * is enqueued; there is no fallback path and no partial mode.  Device-resident
 * index arrays (cu_seqlens, state_idx, the pool slot arrays) are not read by the host: the kernels
 * clamp what they read so that a malformed array cannot make them access memory
 * outside the buffers described by `gdn_dims`, but the results for such input
 * are unspecified.
 */
#ifndef GDN_MI355X_H
#define GDN_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,       /* negative or inconsistent sizes, hv % hk != 0, dv % 16 != 0 */
    GDN_ERR_DTYPE = 3,       /* io_dtype is not GDN_F32 or GDN_BF16 */
    GDN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    GDN_ERR_ALIAS = 5,       /* an output overlaps an input, or h0/hT partially overlap */
    GDN_ERR_UNSUPPORTED = 6, /* dk not in {16, 32, 64, 128}, or a launch-plan request that does not fit */
    GDN_ERR_HIP = 7,         /* the HIP runtime refused the launch */
    GDN_ERR_CAPACITY = 8     /* gdn_bwd_varlen_noalloc: the call needs more than its fixed scratch */
} gdn_status;

typedef enum gdn_dtype {
    GDN_F32 = 0,   /* q, k, v, out are fp32 */
    GDN_BF16 = 1   /* q, k, v, out are bf16; out is rounded to nearest even */
} gdn_dtype;

/*
 * Fused preprocessing (optional, through gdn_dims.pre; NULL means none).  These
 * are the steps the gated delta rule layer runs right before the recurrence
 * (Yang, Kautz, Hatamizadeh, ICLR 2025): L2-normalised queries and keys, a decay
 * exp(g) with g = -exp(A_log) softplus(a + dt_bias) and a write strength
 * beta = sigmoid(b).  The page "Defending Against the Training-Inference Numeric
 * Mismatch in RL (Especially Linear Attention)" (section 3.1) keeps A_log in fp32,
 * as here.  Done inside the kernels they cost no extra pass over HBM, and they
 * are evaluated by one fixed sequence of fp32 operations in every kernel, so the
 * bitwise contract covers them too.
 *
 *   GDN_PRE_QK_L2NORM   every query and key row x (dk values) is replaced by
 *                       x * rsqrt(sum_i x_i^2 + eps) before use, in fp32
 *                       (sum over leaves of 4 consecutive columns, pairwise).
 *   GDN_PRE_GATE_LOGITS the `g` argument holds logits a and the `beta` argument
 *                       logits b (fp32, [T][hv]); the kernels form
 *                       g = -exp(A_log[h]) * softplus(a + dt_bias[h]) and
 *                       beta = sigmoid(b), with softplus(x) = max(x, 0) +
 *                       log1p(exp(-|x|)) evaluated to a few fp32 ulps over the
 *                       whole range (no cut-off for large or very negative x).
 */
enum { GDN_PRE_QK_L2NORM = 1, GDN_PRE_GATE_LOGITS = 2 };

typedef struct gdn_preproc {
    int32_t flags;          /* GDN_PRE_* bits */
    float eps;              /* added to the sum of squares (finite, >= 0; 1e-6 is usual) */
    const float *A_log;     /* [hv] fp32 device; required with GDN_PRE_GATE_LOGITS */
    const float *dt_bias;   /* [hv] fp32 device, or NULL for zero */
} gdn_preproc;

typedef struct gdn_dims {
    int32_t n_seqs;        /* N sequences (prefill) or B decode rows; 0 is a no-op */
    int32_t hk;            /* query/key heads */
    int32_t hv;            /* value heads, a multiple of hk */
    int32_t dk;            /* key/query head dim: 16, 32, 64 or 128 */
    int32_t dv;            /* value head dim: a positive multiple of 16 */
    int32_t io_dtype;      /* gdn_dtype of q, k, v, out */
    int64_t total_tokens;  /* T: rows of q/k/v/g/beta/out; decode requires T == n_seqs */
    int32_t pool_size;     /* P: state pool entries (decode only; ignored by prefill) */
    int32_t plan_lanes;    /* launch shape: lanes holding one state row, 0 = automatic, else 4, 8 or 16 */
    int32_t plan_rows;     /* launch shape: state rows per lane, 0 = automatic, else 1, 2 or 4 */
    int32_t plan_waves;    /* launch shape: waves per workgroup, 0 = automatic, else 1, 2, 4 or 8 */
    int32_t reserved;      /* must be 0 */
    const gdn_preproc *pre; /* fused preprocessing, or NULL (host memory, read during the call) */
} gdn_dims;
/* plan_lanes / plan_rows / plan_waves choose how state rows are spread over
 * lanes, waves and workgroups.  They never change a single bit of any result
 * (every row's arithmetic is fixed, see gdn_fwd_varlen); they exist so that this
 * can be tested and so that a caller can tune the launch.  A field left at 0 is
 * chosen by the library; a combination that is not compiled, or whose rows per
 * workgroup (64 / lanes * rows * waves) do not divide dv, is GDN_ERR_UNSUPPORTED.
 * gdn_decode_step uses plan_rows / plan_waves and always 4 lanes per row. */

/*
 * Varlen prefill: run every sequence of a packed batch through the recurrence.
 *
 *   q, k, v, g, beta : inputs (layouts above); may be NULL only when T == 0
 *   h0               : initial states [N][hv][dv][dk], or NULL for the zero state
 *   cu_seqlens       : [N+1] device int32, cu[0] = 0, non-decreasing, cu[N] = T
 *   out              : [T][hv][dv] outputs o_t (written for every token)
 *   hT               : final states [N][hv][dv][dk], or NULL to skip writing them.
 *                      hT == h0 (the same pointer) updates the states in place;
 *                      any other overlap of the two is GDN_ERR_ALIAS.
 * A sequence of length 0 writes no output and hands h0 (or zeros) to hT.
 */
gdn_status gdn_fwd_varlen(const gdn_dims *dims,
                          const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *h0, const int32_t *cu_seqlens,
                          void *out, float *hT, void *stream);

/*
 * Training forward: gdn_fwd_varlen that also writes saved_p [T][hv][dv] fp32, the
 * key read-out p_t = S_{t-1} k_t of every token and row (the value the recurrence
 * forms for u_t), for gdn_bwd_varlen.  out and hT are bit-identical to
 * gdn_fwd_varlen's.  dims->pre must be NULL (GDN_ERR_UNSUPPORTED); saved_p may be
 * NULL only when T == 0 and must not overlap any other argument.
 */
gdn_status gdn_fwd_varlen_train(const gdn_dims *dims,
                                const void *q, const void *k, const void *v,
                                const float *g, const float *beta,
                                const float *h0, const int32_t *cu_seqlens,
                                void *out, float *hT, float *saved_p, void *stream);

/*
 * Varlen prefill against a state pool, for prefix caching.  The state handling
 * follows what the page "Defending Against the Training-Inference Numeric
 * Mismatch in RL (Especially Linear Attention)" (section 3.2, "Solution") keeps
 * from its serving stack: the recurrent state lives in a cache of slots, and in
 * that stack's "align" cache mode the state is also saved at block-aligned
 * token positions so that a later request sharing the prefix can resume from it.
 *
 * Same operation, inputs, outputs and bitwise contract as gdn_fwd_varlen; only
 * where states come from and go to differs.  P = dims->pool_size (> 0).
 *
 *   state_pool   : [P][hv][dv][dk] fp32, read and written in place
 *   src_idx      : [N] device int32, or NULL.  Sequence n starts from slot
 *                  src_idx[n]; an entry outside [0, P) means the zero state.
 *                  NULL means slot n (then P >= N is required).
 *   dst_idx      : [N] device int32, or NULL.  The final state of sequence n goes
 *                  to slot dst_idx[n]; an entry outside [0, P) means it is not
 *                  written.  NULL means slot n (then P >= N is required).
 *   pos0         : [N] device int32, or NULL (all 0): tokens of sequence n that
 *                  earlier calls already processed.  Used only to place snapshots.
 *   snap_block   : 0 (no snapshots), or a positive multiple of 16.
 *   snap_idx     : [N][snap_per_seq] device int32 (required when snap_block > 0).
 *                  Sequence n's snapshot j is the state after the token that brings
 *                  its absolute position (pos0[n] + tokens done in this call) to the
 *                  j-th multiple of snap_block above pos0[n]; it is stored to slot
 *                  snap_idx[n * snap_per_seq + j], or skipped when that entry is
 *                  outside [0, P) or j >= snap_per_seq.  A snapshot holds exactly
 *                  the bits that hT would hold for a call ending at that token.
 *   out          : [T][hv][dv] outputs, as in gdn_fwd_varlen.
 *
 * Slots written by a call (dst and snapshot entries) must differ from each other
 * and from the slots other sequences of the same call read; a sequence may write
 * the slot it reads from (in place).  These device-side conditions are not
 * checked; breaking them gives unspecified results but no access outside the pool.
 * Errors: as gdn_fwd_varlen, plus GDN_ERR_SHAPE for P <= 0, a bad snap_block or
 * snap_per_seq, or NULL src_idx / dst_idx with P < N; GDN_ERR_NULL for a NULL
 * pool, or NULL snap_idx with snap_block > 0; GDN_ERR_ALIAS when out or the pool
 * overlaps another argument.
 */
gdn_status gdn_fwd_varlen_pool(const gdn_dims *dims,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const int32_t *cu_seqlens, float *state_pool,
                               const int32_t *src_idx, const int32_t *dst_idx,
                               const int32_t *pos0, const int32_t *snap_idx,
                               int32_t snap_block, int32_t snap_per_seq,
                               void *out, void *stream);

/*
 * Decode step: one token for each of B sequences, against states held in a pool
 * and updated in place.  The page "Defending Against the Training-Inference
 * Numeric Mismatch in RL (Especially Linear Attention)" (section 3.2, "Solution")
 * runs decode on the same recurrent kernel as prefill and the trainer's
 * recompute, over the recurrent state its serving stack keeps per request; this
 * is that step, with the pool standing for that state cache.
 *
 *   q, k, v, g, beta : this step's token of each sequence; q, k [B][hk][dk],
 *                      v [B][hv][dv], g, beta [B][hv]   (dims->total_tokens == B)
 *   state_pool       : [P][hv][dv][dk] fp32, read and written in place
 *   state_idx        : [B] device int32: row b uses pool entry state_idx[b];
 *                      NULL means entry b.  Entries must be distinct.  An entry
 *                      outside [0, P) marks a padding row: its output is written
 *                      as zeros and no state is read or written.
 *   out              : [B][hv][dv] outputs
 * The arithmetic is the one of gdn_fwd_varlen for a single token, bit for bit.
 */
gdn_status gdn_decode_step(const gdn_dims *dims,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state_pool, const int32_t *state_idx,
                           void *out, void *stream);

/*
 * Launch shape query (host only: no device memory is read and nothing is enqueued).
 * Runs the same dimension checks and launch planning as gdn_fwd_varlen (decode = 0)
 * or gdn_decode_step (decode != 0) for *dims, and on GDN_OK writes the shape that
 * call would use to shape[0..2] = {lanes per state row, rows per lane, waves per
 * workgroup}.  Pointer checks are not part of it.  shape may not be NULL.
 */
gdn_status gdn_query_plan(const gdn_dims *dims, int32_t decode, int32_t *shape);

/*
 * Short causal convolution with a carried state (the step that feeds the
 * recurrence its q, k and v).  For every sequence n, channel c and token t of the
 * sequence, with K taps:
 *
 *     z = bias[c] + sum_{j=0}^{K-1} w[c][j] * x(t - (K-1) + j, c)      (fp32, j ascending, fma)
 *     y[t][c] = z * sigmoid(z)   (GDN_CONV_SILU; else y = z), rounded to the io dtype
 *
 * where x(s, c) for s before the sequence's first token is read from the
 * sequence's state: state[slot][c][m] is the input m - (K-1) tokens before the
 * first token (oldest first).  Afterwards the state slot holds the sequence's
 * last K-1 inputs (reaching back into the old state for sequences shorter than
 * K-1).  Every output depends only on its own sequence's inputs, so the bitwise
 * contract holds: a decode step is a call whose sequences have one token each,
 * and cutting a sequence into calls that carry the state gives the same bits.
 * The page "Defending Against the Training-Inference Numeric Mismatch in RL
 * (Especially Linear Attention)" (section 3.2, "Solution") keeps this conv state
 * in the serving stack's cache beside the recurrent state.
 *
 *   x, y        : [T][C] io dtype (y is written for every token)
 *   w           : [C][K] fp32;  bias: [C] fp32 or NULL
 *   cu_seqlens  : [N+1] device int32, as for gdn_fwd_varlen
 *   state_pool  : [P][C][K-1] io dtype, read and written in place
 *   src_idx / dst_idx : [N] device int32 or NULL (slot n, then P >= N).  An entry
 *                 outside [0, P) means the zero state / no write.  The same slot
 *                 may be read and written by one sequence (in place); a slot
 *                 written for one sequence must not be read or written for
 *                 another in the same call.
 * Errors: NULL, SHAPE (K outside 2..8, C <= 0 or not a multiple of 16 bytes of
 * elements (8 bf16, 4 fp32), P <= 0, P < N without index arrays, T inconsistent),
 * DTYPE, ALIGN (x, y, state 16 bytes; w, bias, indices 4 bytes),
 * ALIAS (y or the pool overlapping another argument).
 */
enum { GDN_CONV_SILU = 1 };

typedef struct gdn_conv_dims {
    int32_t n_seqs;        /* N; 0 is a no-op */
    int32_t channels;      /* C */
    int32_t taps;          /* K, 2 .. 8 */
    int32_t io_dtype;      /* gdn_dtype of x, y and the state pool */
    int64_t total_tokens;  /* T */
    int32_t pool_size;     /* P */
    int32_t flags;         /* GDN_CONV_* bits */
} gdn_conv_dims;

gdn_status gdn_short_conv(const gdn_conv_dims *dims, const void *x, const float *w, const float *bias,
                          const int32_t *cu_seqlens, void *state_pool, const int32_t *src_idx,
                          const int32_t *dst_idx, void *y, void *stream);

/*
 * Backward of gdn_short_conv: given dy = dL/dy (fp32 [T][C]), the gradients of the
 * inputs x, the taps w, the bias and the carried state the call read, with z
 * recomputed exactly as the forward forms it:
 *
 *     dz(t)    = dy(t) sigmoid(z) (1 + z (1 - sigmoid(z)))   (GDN_CONV_SILU; else dy)
 *     dx(s)    = sum_{i=0}^{K-1} w[c][K-1-i] dz(s + i)       (s's own sequence only)
 *     dw[c][j] = sum_t dz(t) x(t - (K-1) + j),   dbias[c] = sum_t dz(t)
 *     dstate[n][c][m] = sum_{j <= m} w[c][j] dz(t_n + m - j)  (t_n: sequence n's first token)
 *
 * dw and dbias sum over every token of the call (a partial sum per 64-token
 * block; per channel, four quarters of the blocks each added in block order, then
 * (q0 + q1) + (q2 + q3)); everything else is per sequence.  The state written by the
 * forward is a copy of inputs for the next call, not differentiated here.
 *
 *   x, w, bias, cu_seqlens, src_idx : as gdn_short_conv
 *   state_pool  : [P][C][K-1] io dtype, the states the forward read (keep them if
 *                 the forward updated its slots in place)
 *   dx          : [T][C] fp32;  dw: [C][K] fp32;  dbias: [C] fp32 or NULL;
 *   dstate      : [N][C][K-1] fp32 or NULL
 *   workspace   : device scratch of gdn_short_conv_backward_workspace_size bytes
 *                 (4 (K+1) C bytes per 64 tokens), 4-byte aligned; contents on
 *                 entry do not matter.
 * Errors: NULL, SHAPE (K outside 2..8, C <= 0, P <= 0, P < N without src_idx, a
 * small workspace), DTYPE, UNSUPPORTED (unknown flags), ALIGN (x and the pool to
 * their element size, the rest 4 bytes), ALIAS (an output overlapping an input or
 * another output).
 */
gdn_status gdn_short_conv_backward_workspace_size(const gdn_conv_dims *dims, uint64_t *bytes);

gdn_status gdn_short_conv_backward(const gdn_conv_dims *dims, const void *x, const float *w, const float *bias,
                                   const int32_t *cu_seqlens, const void *state_pool, const int32_t *src_idx,
                                   const float *dy, float *dx, float *dw, float *dbias, float *dstate,
                                   void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * Backward of gdn_fwd_varlen: gradients of a loss L with respect to every input,
 * given dL/dout and (optionally) dL/dhT.  The page "Defending Against the
 * Training-Inference Numeric Mismatch in RL (Especially Linear Attention)"
 * (section 3.2) runs the recurrence in every forward and leaves the trainer's
 * backward to a separate kernel; this is that backward for the same recurrence.
 * With p_t = S_{t-1} k_t and u_t = beta_t (v_t - a_t p_t) (so S_t = a_t S_{t-1} +
 * u_t k_t^T), and D_t = dL/dS_t walked from the last token back
 * (D <- D + dO_t q_t^T, du_t = D k_t, D <- a_t (D - beta_t du_t k_t^T)):
 *
 *     dq_t = S_t^T dO_t                 dk_t = D_t^T u_t - a_t beta_t S_{t-1}^T du_t
 *     dv_t = beta_t du_t                dbeta_t = du_t . (v_t - a_t p_t)
 *     dg_t = <dhT, hT> + sum_{s >= t in the sequence} (dO_s . o_s - dv_s . v_s)
 *     dh0  = D_0
 *
 * dq and dk of a key head add up the value heads that read it.  All sums have a
 * fixed order and nothing crosses sequences, so the gradients are deterministic
 * and do not depend on the batch; they are fp32 computations, not bitwise equal
 * to any other path.
 *
 *   q, k, v, g, beta, h0, cu_seqlens : the forward's inputs (dims->pre must be NULL)
 *   dout        : [T][hv][dv] io dtype, dL/dout
 *   dhT         : [N][hv][dv][dk] fp32, dL/dhT, or NULL for zero
 *   saved_p     : p_t from gdn_fwd_varlen_train on the same inputs, or NULL.  Given, the
 *                 backward skips its own forward recompute (one of its four passes).
 *   hT          : the forward's final states; required when saved_p and dhT are both
 *                 given (for <dhT, hT>), otherwise ignored and may be NULL
 *   dq, dk      : [T][hk][dk] fp32 outputs
 *   dv          : [T][hv][dv] fp32 output
 *   dg, dbeta   : [T][hv] fp32 outputs
 *   dh0         : [N][hv][dv][dk] fp32 output, or NULL to skip it
 *   workspace   : device scratch of at least gdn_bwd_workspace_size bytes, 16-byte
 *                 aligned, owned by the caller; its contents on entry do not matter
 * dk and dv must each be 32, 64 or 128 (else GDN_ERR_UNSUPPORTED, as are a set
 * dims->pre and plan fields).  Outputs and workspace must not overlap each other
 * or an input (GDN_ERR_ALIAS); a workspace smaller than needed is GDN_ERR_SHAPE.
 */
gdn_status gdn_bwd_workspace_size(const gdn_dims *dims, uint64_t *bytes);

gdn_status gdn_bwd_varlen(const gdn_dims *dims,
                          const void *q, const void *k, const void *v,
                          const float *g, const float *beta,
                          const float *h0, const int32_t *cu_seqlens,
                          const void *dout, const float *dhT,
                          const float *saved_p, const float *hT,
                          float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dh0,
                          void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * Allocation-free backward, for callers that cannot allocate or pass device
 * memory during the call: code under HIP graph capture, tight serving or training
 * loops, and harnesses that forbid allocation.  Same operation, arguments (minus
 * the workspace), checks and bits as gdn_bwd_varlen; the workspace is instead a
 * fixed array of GDN_NOALLOC_SCRATCH_BYTES (64 MiB) in device memory, one per
 * device, which that device holds until the process ends.  The call allocates
 * nothing and calls no allocating routine; its first call on a device looks up
 * the array's address (hipGetSymbolAddress) and keeps it.
 *
 * Capacity: the call needs gdn_bwd_workspace_size(dims) bytes of it, about
 * 8 hv (dk + dv) bytes per token plus 4 hv dv dk bytes per sequence (64 KiB per
 * token and 2 MiB per sequence at hv = 32, dk = dv = 128: about 990 tokens for one
 * sequence); a call that needs more returns GDN_ERR_CAPACITY before anything
 * touches the device.
 *
 * Every call on one device shares that device's array: calls on one device that
 * may overlap in time (different streams, or host threads without ordering) race
 * on it and give unspecified gradients; calls ordered on one stream are safe.  The
 * array's contents on entry do not matter (the backward overwrites what it reads).
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64ull << 20)

gdn_status gdn_bwd_varlen_noalloc(const gdn_dims *dims,
                                  const void *q, const void *k, const void *v,
                                  const float *g, const float *beta,
                                  const float *h0, const int32_t *cu_seqlens,
                                  const void *dout, const float *dhT,
                                  const float *saved_p, const float *hT,
                                  float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dh0,
                                  void *stream);

/*
 * Chunked form with a replaying decode.  gdn_fwd_varlen and gdn_decode_step make
 * decode match prefill by running token by token everywhere, as the page
 * "Defending Against the Training-Inference Numeric Mismatch in RL (Especially
 * Linear Attention)" (section 3.2) does.  The other way, in the summary of
 * "Finish RL Training Faster: Bitwise-Consistent, High-Performance, Agent-Driven"
 * (section "Consistency has several layers"), keeps a chunked prefill and has
 * decode replay its computation order; that needs chunk boundaries that do not
 * move, since a recurrent state carries where it was cut (the bitwise-parity post
 * on linear attention, "Why linear attention is the next wall").
 * Here chunks are the 16-token stretches at positions 16c .. 16c+15 of a
 * sequence.  Within a chunk, with S0 its starting state, a_m = exp(g_m),
 * Gam_{m,r} = a_m a_{m-1} .. a_{r+1} (1 for r = m), Gam_m = Gam_{m,0} a_0,
 * A[m][r] = beta_m Gam_{m,r} (k_m . k_r) (r < m) and T = (I + A)^-1:
 *
 *   R_m = beta_m (v_m - Gam_m S0 k_m),   U = T R   (u_m = R_m - sum_{r<m} A[m][r] u_r)
 *   o_m = Gam_m S0 q_m + sum_{s<=m} Gam_{m,s} (q_m . k_s) u_s
 *   chunk end:  S = Gam_15 S0 + sum_s Gam_{15,s} u_s k_s^T
 *
 * (the same rule as gdn_fwd_varlen, written from the chunk's start; results
 * agree with it to rounding, not bitwise).  Every product runs on the matrix cores
 * (fp32 MFMA, fp32 accumulation).  Each token's results depend only on S0 and its
 * chunk's tokens up to it (later tokens enter only as exact zero products, and +0
 * is added so a zero result has one sign), so the state between calls is a
 * gdn_chunk_state, and every split of a sequence into calls -- a decode step of
 * one token included -- gives the same bits, as do batch-mates and batch order.
 * Non-finite inputs are the exception: since 0 x NaN is NaN, a NaN or infinity in
 * a token reaches the outputs of its whole 16-token chunk (never an earlier chunk
 * or another sequence), and a decode step, which has not seen the later tokens,
 * then differs from a prefill of the chunk.
 *
 *   in   : the sequences' chunked states, or NULL for empty ones (zero state, no
 *          open chunk).  A state with S = h0 and count = 0 starts from h0.
 *   out  : where the new chunked states go (all six arrays).  out may share S, k,
 *          r, a and b with in (the same five pointers: an in-place update, which
 *          then writes S only when a chunk closes) when every sequence of the call
 *          has exactly one token (total_tokens == n_seqs, a decode step); the count
 *          arrays must always differ.  Any other overlap is GDN_ERR_ALIAS.
 *   o    : [T][hv][dv] outputs, io dtype.
 *   cu_seqlens : as for gdn_fwd_varlen, or NULL when T == N: then sequence n's one
 *          token is row n, the results are those of cu_seqlens = 0, 1, .., N, and
 *          a single kernel does the step (GDN_ERR_NULL if T != N).
 *   workspace : device scratch of at least gdn_chunked_workspace_size bytes,
 *          16-byte aligned, owned by the caller; its contents on entry do not
 *          matter.  About 2.3 KB per (chunk touched, value head).
 * dk must be 64 or 128, dv a multiple of 16 and hv / hk at most 16 (else
 * GDN_ERR_UNSUPPORTED, as are dims->pre, plan_lanes and plan_rows).  plan_waves (0 = automatic, else 1, 2 or
 * 4) is how many waves share one 16-row state tile, each holding a part of its
 * dk columns; it never changes a bit.  Errors as gdn_fwd_varlen (S and k of both
 * states 16-byte aligned; r, a, b, count 4-byte); a count outside 0..15 is clamped
 * on the device.
 */
enum { GDN_CHUNK = 16 };

typedef struct gdn_chunk_state {
    float *S;        /* [N][hv][dv][dk] fp32: state at the start of the open chunk */
    float *k;        /* [N][16][hk][dk] fp32: keys of the open chunk's tokens */
    float *r;        /* [N][16][hv][dv] fp32: their R rows beta (v - Gam S0 k) */
    float *a;        /* [N][16][hv]     fp32: their decay factors exp(g) */
    float *b;        /* [N][16][hv]     fp32: their betas */
    int32_t *count;  /* [N]             tokens in the open chunk, 0 .. 15 */
} gdn_chunk_state;

gdn_status gdn_chunked_workspace_size(const gdn_dims *dims, uint64_t *bytes);

gdn_status gdn_fwd_chunked(const gdn_dims *dims,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const int32_t *cu_seqlens,
                           const gdn_chunk_state *in, const gdn_chunk_state *out,
                           void *o, void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * Chunked backward: the gradients of gdn_bwd_varlen (same operation, inputs and
 * outputs; dims->pre must be NULL) taken chunk by chunk on the matrix cores.  The
 * page "Defending Against the Training-Inference Numeric Mismatch in RL (Especially
 * Linear Attention)" (section 3.2, "Solution") keeps every forward on the recurrent
 * kernel and the chunked kernel for the training backward; this is that backward,
 * for the recurrence gdn_fwd_varlen computes.
 *
 * In the notation of gdn_fwd_chunked (chunks at positions 16c .. 16c+15, l the
 * chunk's last token, x_m = v_m - Gam_m S0 k_m, U = T (beta x)), with D = dL/dS
 * after the chunk and dO its output gradients, a chunk contributes
 *
 *   dU = B^T dO + Gam_{l,.} (K D^T),   dR = T^T dU,   dv = beta dR,
 *   dB = dO U^T,  dA = -dR U^T,  H[m][r] = dA[m][r] beta_m Gam_{m,r}  (r < m),
 *   dq_m  = Gam_m S0^T dO_m + sum_{s<=m} dB[m][s] Gam_{m,s} k_s,
 *   dk_s  = -beta_s Gam_s S0^T dR_s + Gam_{l,s} D^T u_s + sum_{m>=s} dB[m][s] Gam_{m,s} q_m
 *           + sum_r (H[s][r] + H[r][s]) k_r,
 *   dbeta_m = dR_m . x_m + sum_{r<m} dA[m][r] Gam_{m,r} (k_m . k_r),
 *   D at the chunk's start = Gam_l D + sum_m Gam_m dO_m q_m^T - sum_m beta_m Gam_m dR_m k_m^T,
 *
 * dg as in gdn_bwd_varlen (<dhT, hT> plus the reverse sum of dO . o - dv . v) and
 * dh0 = D at the sequence's start.  A forward walk over the chunks first stores
 * the state at every chunk's start in the workspace; P workgroups per sequence and
 * value head, each holding dv/P rows of D, then walk the chunks backwards, and
 * the parts' shares of the sums over rows (dq, dk, dbeta, dg) are added in order
 * afterwards.  Every sum has a fixed order and nothing crosses sequences: the
 * gradients are deterministic and do not depend on the batch (fp32 computations,
 * equal to gdn_bwd_varlen's to rounding, not bitwise; P = 1 and P = 2 round
 * differently).
 *
 *   workspace : device scratch of at least gdn_bwd_chunked_workspace_size bytes,
 *               16-byte aligned, owned by the caller; contents on entry do not
 *               matter.  About 4 dv (dk + 16) bytes per (16-token chunk, value head)
 *               for the chunk-start states and x, plus 4 hv (2 P dk + 2 P) bytes per
 *               token (the dk term only when hv > hk or P > 1, the last when P > 1)
 *               and 4.3 KB per (chunk, value head).
 * dk must be 64 or 128, dv 32, 64 or 128 and hv / hk at most 16 (else
 * GDN_ERR_UNSUPPORTED, as is dims->pre).  plan_rows sets P (0 = automatic: 2 for
 * dv = 128, else 1; 2 needs dv >= 64), plan_waves (0, 1, 2 or 4) the forward
 * walk's waves per 16-row tile, and plan_lanes 0 (automatic) or 1 (the plain
 * reverse walk: for dv = 128 in two parts the automatic choice overlaps the
 * chunk-recurrence waves of one chunk with the gradient waves of the next); the
 * waves and the reverse walk's form change no bit.  plan_lanes above 1 is
 * GDN_ERR_UNSUPPORTED.  Other errors as gdn_bwd_varlen.
 */
gdn_status gdn_bwd_chunked_workspace_size(const gdn_dims *dims, uint64_t *bytes);

gdn_status gdn_bwd_chunked(const gdn_dims *dims,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           const float *h0, const int32_t *cu_seqlens,
                           const void *dout, const float *dhT,
                           float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dh0,
                           void *workspace, uint64_t workspace_bytes, void *stream);

/*
 * The fused preprocessing as a pass of its own, and its gradients: what a trainer
 * needs to differentiate through the layer's preprocessing (the gated delta rule
 * layer of Yang, Kautz, Hatamizadeh, ICLR 2025; A_log kept in fp32 as in the page
 * "Defending Against the Training-Inference Numeric Mismatch in RL (Especially
 * Linear Attention)", section 3.1).  With dims->pre (or NULL: no preprocessing):
 *
 *   gdn_preprocess: qn, kn = the L2-normalised q, k rows (fp32 [T][hk][dk]) and
 *     g, beta (fp32 [T][hv]) from the logits a, b, each by the fp32 operations the
 *     fused kernels use (see gdn_preproc above), so that gdn_fwd_varlen with
 *     io_dtype GDN_F32 on (qn, kn, v widened, g, beta) computes the fused call's
 *     state bit for bit and its outputs before their rounding to bf16.
 *   gdn_preprocess_backward: given dL/dqn, dL/dkn, dL/dg and dL/dbeta (fp32, e.g.
 *     from gdn_bwd_varlen or gdn_bwd_chunked on the preprocessed values), the
 *     gradients of the raw inputs:
 *       dq = (dqn - qn (qn . dqn)) r with r = rsq(sum q^2 + eps) (likewise dk);
 *       da = dg (-exp(A_log) sigmoid(a + dt_bias));  db = dbeta beta (1 - beta);
 *       dA_log[h] = sum_t dg g;  ddt_bias[h] = sum_t da  (all T tokens, fixed order:
 *       64-token blocks, then the blocks; da and db hold the block sums until
 *       they are overwritten with their own values, within the call)
 *     Without GDN_PRE_QK_L2NORM dq = dqn (dk = dkn); without GDN_PRE_GATE_LOGITS
 *     da = dg, db = dbeta and dA_log, ddt_bias are not written; ddt_bias is written
 *     only when pre->dt_bias is given.
 *
 *   q, k : [T][hk][dk] io dtype, 16-byte aligned; a, b, g, beta, da, db, dg, dbeta:
 *          [T][hv] fp32; qn, kn, dqn, dkn, dq, dk: [T][hk][dk] fp32, 16-byte aligned;
 *          dA_log, ddt_bias: [hv] fp32.  All device memory, owned by the caller.
 * Only hk, hv, dk (16, 32, 64 or 128), dv, io_dtype, total_tokens and pre of dims
 * are used (n_seqs is not).  Errors as gdn_fwd_varlen: NULL, SHAPE (also a call
 * whose launch grids would pass 2^31 workgroups), DTYPE, UNSUPPORTED, ALIGN, ALIAS
 * (an output overlapping an input or another output).
 */
gdn_status gdn_preprocess(const gdn_dims *dims, const void *q, const void *k, const float *a, const float *b,
                          float *qn, float *kn, float *g, float *beta, void *stream);

gdn_status gdn_preprocess_backward(const gdn_dims *dims, const void *q, const void *k, const float *a,
                                   const float *b, const float *dqn, const float *dkn, const float *dg,
                                   const float *dbeta, float *dq, float *dk, float *da, float *db, float *dA_log,
                                   float *ddt_bias, void *stream);

/* Human-readable description of a status code (static storage; an unknown code
 * gives "unknown gdn_status").  Every refusal is reported as one of these codes rather than
 * served by another, non-invariant path: the bitwise-parity post on linear
 * attention ("Why linear attention is the next wall") describes a serving stack
 * that refuses batch-invariant mode outright, with no fallback and no partial
 * mode, when a kernel cannot honour it, and this library keeps that convention. */
const char *gdn_status_string(gdn_status status);

/* ABI version of this header (major * 100 + minor). */
int32_t gdn_abi_version(void);

#define GDN_ABI_VERSION 210

#ifdef __cplusplus
}
#endif

#endif /* GDN_MI355X_H */
