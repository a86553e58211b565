/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet recurrent forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (per sequence n, per value head h):
 *
 *   S_0 = h0[n][h]  (or 0)
 *   for t over the tokens of sequence n, in order:
 *     a_t = exp(g[t][h])
 *     S  <- a_t * S                                  (decay the previous state)
 *     u_j = beta[t][h] * (v[t][h][j] - sum_i S[j][i] k[t][hk][i])
 *     S[j][i] <- S[j][i] + u_j * k[t][hk][i]         (delta-rule write)
 *     o[t][h][j] = sum_i S[j][i] q[t][hk][i]         (read-out of the new state)
 *   hT[n][h] = S
 *
 * which is the gated delta rule S_t = a_t S_{t-1} (I - beta_t k_t k_t^T)
 * + beta_t v_t k_t^T, o_t = S_t q_t (Yang, Kautz, Hatamizadeh, "Gated Delta
 * Networks: Improving Mamba2 with Delta Rule", ICLR 2025, the gated delta rule
 * equation), with the state stored as a dv x dk matrix S[j][i] so that S k is a
 * dv-vector.  The token-by-token walk of one sequence against that sequence's
 * own state, with nothing shared across sequences, is the "recurrent kernel" of
 * the page "Defending Against the Training-Inference Numeric Mismatch in RL
 * (Especially Linear Attention)", section 3.2 (Operator level: linear attention).
 * The fp32 state and bf16 forward precision recipe are that page's set-up tables
 * (section 4.2.1); the oracle itself works in fp64 on the exact fp32 values of
 * the inputs.
 *
 * Value head h reads query/key head h / (hv / hk) (grouped heads: consecutive
 * value heads share one key head).  No 1/sqrt(dk) scale is applied to q.
 *
 * Layouts (all contiguous, token-major):
 *   q, k   : [T][hk][dk]   qk_dtype: fp32 (0), bf16 bits (1) or fp64 (2)
 *   v      : [T][hv][dv]   v_dtype, same codes
 *   g, beta: [T][hv]       gate_dtype: fp32 (0) or fp64 (2)
 *   h0, hT : [N][hv][dv][dk] fp64 (h0 may be NULL = zero state, hT may be NULL)
 *   out    : [T][hv][dv]   fp64
 *   cu_seqlens: [N+1] int32, cu[0] = 0, non-decreasing, cu[N] = T.
 *
 * Parallelism: OpenMP over independent (sequence, value head) units only; the
 * arithmetic inside a unit is the sequential loop above.
 *
 * gdn_oracle_preprocess (below) forms q, k, g and beta from the raw inputs of the
 * fused path in fp64; its results feed gdn_oracle_forward with dtype code 2.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of one input element to double. */
static double oracle_load(const void *base, int64_t idx, int io_dtype)
{
    if (io_dtype == 0)
        return (double)((const float *)base)[idx];
    if (io_dtype == 2)
        return ((const double *)base)[idx];
    /* bf16 is the top half of an IEEE binary32; the widening is exact. */
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Returns 0 on success, a negative value on a bad argument. */
int gdn_oracle_forward(int32_t n_seqs, const int32_t *cu_seqlens,
                       int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                       int32_t qk_dtype, int32_t v_dtype, int32_t gate_dtype,
                       const void *q, const void *k, const void *v,
                       const void *g, const void *beta,
                       const double *h0, double *out, double *hT,
                       int32_t n_threads)
{
    if (n_seqs < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (hv % hk != 0)
        return -2;
    if (qk_dtype < 0 || qk_dtype > 2 || v_dtype < 0 || v_dtype > 2 || (gate_dtype != 0 && gate_dtype != 2))
        return -3;
    if (n_seqs == 0)
        return 0;
    if (!cu_seqlens || !g || !beta || !out)
        return -4;
    for (int32_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -5;
    if (cu_seqlens[0] != 0)
        return -5;
    const int64_t total = cu_seqlens[n_seqs];
    if (total > 0 && (!q || !k || !v))
        return -4;

    const int32_t group = hv / hk;
    const int64_t n_units = (int64_t)n_seqs * hv;
    int status = 0;
    if (n_threads <= 0)
        n_threads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t unit = 0; unit < n_units; ++unit) {
        const int32_t n = (int32_t)(unit / hv);
        const int32_t h = (int32_t)(unit % hv);
        const int32_t kh = h / group;
        double *S = (double *)malloc(sizeof(double) * (size_t)dv * (size_t)dk);
        if (!S) {
#pragma omp atomic write
            status = -6;
            continue;
        }
        const size_t state_off = ((size_t)n * hv + h) * (size_t)dv * (size_t)dk;
        for (int64_t e = 0; e < (int64_t)dv * dk; ++e)
            S[e] = h0 ? h0[state_off + e] : 0.0;

        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const double a = exp(oracle_load(g, t * hv + h, gate_dtype));
            const double b = oracle_load(beta, t * hv + h, gate_dtype);
            const int64_t qk_off = (t * hk + kh) * (int64_t)dk;
            const int64_t v_off = (t * hv + h) * (int64_t)dv;

            for (int64_t e = 0; e < (int64_t)dv * dk; ++e)
                S[e] = a * S[e];

            for (int32_t j = 0; j < dv; ++j) {
                double *row = S + (size_t)j * dk;
                double p = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    p += row[i] * oracle_load(k, qk_off + i, qk_dtype);
                const double u = b * (oracle_load(v, v_off + j, v_dtype) - p);
                for (int32_t i = 0; i < dk; ++i)
                    row[i] += u * oracle_load(k, qk_off + i, qk_dtype);
                double o = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    o += row[i] * oracle_load(q, qk_off + i, qk_dtype);
                out[v_off + j] = o;
            }
        }
        if (hT)
            memcpy(hT + state_off, S, sizeof(double) * (size_t)dv * (size_t)dk);
        free(S);
    }
    return status;
}

/*
 * Preprocessing of the fused path, in fp64, from the raw per-token inputs:
 *
 *   q'[t][kh][:] = q[t][kh][:] / sqrt(sum_i q[t][kh][i]^2 + eps)     (same for k)
 *   g[t][h]      = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h]),
 *                  softplus(x) = log(1 + exp(x)), evaluated as log1p(exp(x))
 *   beta[t][h]   = 1 / (1 + exp(-b[t][h]))
 *
 * This is the gate and key/query handling of the gated delta rule layer (Yang,
 * Kautz, Hatamizadeh, ICLR 2025: L2-normalised keys and queries; a Mamba2-style
 * decay exp(-exp(A_log) softplus(.)) and a sigmoid write strength).  The page
 * "Defending Against the Training-Inference Numeric Mismatch in RL (Especially
 * Linear Attention)" (section 3.1) keeps A_log in fp32, as here.
 *
 * q, k: [T][hk][dk] in io_dtype (0 fp32, 1 bf16); a, b: [T][hv] fp32;
 * A_log: [hv] fp32; dt_bias: [hv] fp32 or NULL (zero).  Outputs in fp64:
 * qn, kn: [T][hk][dk]; g, beta: [T][hv].  With norm_qk == 0, qn and kn are the
 * inputs widened; with A_log == NULL, g and beta are a and b widened.
 */
int gdn_oracle_preprocess(int64_t T, int32_t hk, int32_t hv, int32_t dk, int32_t io_dtype,
                          const void *q, const void *k, const float *a, const float *b,
                          const float *A_log, const float *dt_bias, int32_t norm_qk, double eps,
                          double *qn, double *kn, double *g, double *beta)
{
    if (T < 0 || hk <= 0 || hv <= 0 || dk <= 0 || (io_dtype != 0 && io_dtype != 1))
        return -1;
    if (T > 0 && (!q || !k || !a || !b || !qn || !kn || !g || !beta))
        return -4;
    for (int64_t r = 0; r < T * hk; ++r) {
        const int64_t off = r * dk;
        double sq = 0.0, sk = 0.0;
        for (int32_t i = 0; i < dk; ++i) {
            const double x = oracle_load(q, off + i, io_dtype);
            const double y = oracle_load(k, off + i, io_dtype);
            sq += x * x;
            sk += y * y;
        }
        const double dq = norm_qk ? sqrt(sq + eps) : 1.0;
        const double dkn = norm_qk ? sqrt(sk + eps) : 1.0;
        for (int32_t i = 0; i < dk; ++i) {
            qn[off + i] = oracle_load(q, off + i, io_dtype) / dq;
            kn[off + i] = oracle_load(k, off + i, io_dtype) / dkn;
        }
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < hv; ++h) {
            const int64_t i = t * hv + h;
            if (A_log) {
                const double x = (double)a[i] + (dt_bias ? (double)dt_bias[h] : 0.0);
                g[i] = -exp((double)A_log[h]) * log1p(exp(x));
                beta[i] = 1.0 / (1.0 + exp(-(double)b[i]));
            } else {
                g[i] = (double)a[i];
                beta[i] = (double)b[i];
            }
        }
    }
    return 0;
}

/*
 * Short causal convolution of the gated delta rule layer, in fp64: for every
 * sequence n, channel c and token t of the sequence, with K taps,
 *
 *   z[t][c] = bias[c] + sum_{j=0}^{K-1} w[c][j] * x(t - (K-1) + j, c)
 *   y[t][c] = z / (1 + exp(-z))        (SiLU; with silu == 0, y = z)
 *
 * where x(s, c) for s before the sequence's first token is taken from the
 * sequence's convolution state: state[n][c][m] holds the input m - (K-1) tokens
 * before the first token (m = 0 .. K-2, oldest first), or 0 when state is NULL.
 * After the sequence, state_out[n][c][m] = x(last - (K-2) + m, c), i.e. the last
 * K-1 inputs, again oldest first (reaching back into the old state when the
 * sequence is shorter than K-1).  This is the depthwise causal convolution with
 * a carried state that the layer runs on its q, k and v projections (Yang, Kautz,
 * Hatamizadeh, ICLR 2025); the page "Defending Against the Training-Inference
 * Numeric Mismatch in RL (Especially Linear Attention)" (section 3.2, "Solution")
 * keeps that conv state in the serving stack's cache.
 *
 * x: [T][C] in io_dtype (0 fp32, 1 bf16); w: [C][K] fp32; bias: [C] fp32 or NULL;
 * state, state_out: [N][C][K-1] fp64 (either may be NULL); y: [T][C] fp64.
 */
int gdn_oracle_short_conv(int32_t n_seqs, const int32_t *cu_seqlens, int32_t C, int32_t K, int32_t io_dtype,
                          const void *x, const float *w, const float *bias, const double *state,
                          int32_t silu, double *y, double *state_out)
{
    if (n_seqs < 0 || C <= 0 || K < 1 || (io_dtype != 0 && io_dtype != 1))
        return -1;
    if (n_seqs == 0)
        return 0;
    if (!cu_seqlens || !w || (cu_seqlens[n_seqs] > 0 && (!x || !y)))
        return -4;
    const int32_t M = K - 1;
    for (int32_t n = 0; n < n_seqs; ++n) {
        const int64_t tb = cu_seqlens[n], te = cu_seqlens[n + 1];
        if (te < tb)
            return -5;
        for (int32_t c = 0; c < C; ++c) {
            /* x(s, c) for s = tb - M .. te - 1, as a plain array: the old state first */
            const int64_t len = te - tb;
            double *win = (double *)malloc(sizeof(double) * (size_t)(M + len + 1));
            if (!win)
                return -6;
            for (int32_t m = 0; m < M; ++m)
                win[m] = state ? state[((int64_t)n * C + c) * M + m] : 0.0;
            for (int64_t t = 0; t < len; ++t)
                win[M + t] = oracle_load(x, (tb + t) * C + c, io_dtype);
            for (int64_t t = 0; t < len; ++t) {
                double z = bias ? (double)bias[c] : 0.0;
                for (int32_t j = 0; j < K; ++j)
                    z += (double)w[(int64_t)c * K + j] * win[t + j];
                y[(tb + t) * C + c] = silu ? z / (1.0 + exp(-z)) : z;
            }
            if (state_out)
                for (int32_t m = 0; m < M; ++m)
                    state_out[((int64_t)n * C + c) * M + m] = win[len + m];
            free(win);
        }
    }
    return 0;
}

/*
 * Gradients of gdn_oracle_preprocess, in fp64 (reverse mode of each of its maps),
 * given the gradients of a loss with respect to its outputs:
 *
 *   L2 norm, y = x / s with s = sqrt(sum_i x_i^2 + eps):
 *       dL/dx_i = (dL/dy_i) / s - x_i (x . dL/dy) / s^3
 *   gate, g = -exp(A_log) softplus(z) with z = a + dt_bias (softplus' = sigmoid):
 *       dL/da = dL/dg * (-exp(A_log) sigmoid(z)),   dL/dA_log[h] = sum_t dL/dg g,
 *       dL/ddt_bias[h] = sum_t dL/da          (sums over t = 0 .. T-1 in order)
 *   write strength, beta = sigmoid(b):  dL/db = dL/dbeta beta (1 - beta)
 *
 * The maps are those of gdn_oracle_preprocess (normalised keys and queries, the
 * Mamba2-style decay and the sigmoid write strength of the gated delta rule layer,
 * Yang, Kautz, Hatamizadeh, ICLR 2025).  Without norm_qk the first map is the
 * identity (dq = dqn); without A_log the gate and beta maps are identities
 * (da = dg, db = dbeta) and dA_log, ddt_bias are left alone.
 *
 * Inputs as gdn_oracle_preprocess plus dqn, dkn [T][hk][dk] and dg, dbeta [T][hv],
 * fp64.  Outputs, fp64: dq, dk [T][hk][dk]; da, db [T][hv]; dA_log, ddt_bias [hv]
 * (either may be NULL to skip it).
 */
int gdn_oracle_preprocess_backward(int64_t T, int32_t hk, int32_t hv, int32_t dk, int32_t io_dtype,
                                   const void *q, const void *k, const float *a, const float *b,
                                   const float *A_log, const float *dt_bias, int32_t norm_qk, double eps,
                                   const double *dqn, const double *dkn, const double *dg, const double *dbeta,
                                   double *dq, double *dk_out, double *da, double *db,
                                   double *dA_log, double *ddt_bias)
{
    if (T < 0 || hk <= 0 || hv <= 0 || dk <= 0 || (io_dtype != 0 && io_dtype != 1))
        return -1;
    if (T > 0 && (!q || !k || !a || !b || !dqn || !dkn || !dg || !dbeta || !dq || !dk_out || !da || !db))
        return -4;
    for (int64_t r = 0; r < T * hk; ++r) {
        const int64_t off = r * dk;
        for (int side = 0; side < 2; ++side) {
            const void *x = side ? k : q;
            const double *dy = side ? dkn : dqn;
            double *dx = side ? dk_out : dq;
            if (!norm_qk) {
                for (int32_t i = 0; i < dk; ++i)
                    dx[off + i] = dy[off + i];
                continue;
            }
            double ss = 0.0, xdy = 0.0;
            for (int32_t i = 0; i < dk; ++i) {
                const double xi = oracle_load(x, off + i, io_dtype);
                ss += xi * xi;
                xdy += xi * dy[off + i];
            }
            const double s = sqrt(ss + eps);
            for (int32_t i = 0; i < dk; ++i) {
                const double xi = oracle_load(x, off + i, io_dtype);
                dx[off + i] = dy[off + i] / s - xi * xdy / (s * s * s);
            }
        }
    }
    if (A_log) {
        if (dA_log)
            for (int32_t h = 0; h < hv; ++h)
                dA_log[h] = 0.0;
        if (ddt_bias)
            for (int32_t h = 0; h < hv; ++h)
                ddt_bias[h] = 0.0;
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < hv; ++h) {
            const int64_t i = t * hv + h;
            if (!A_log) {
                da[i] = dg[i];
                db[i] = dbeta[i];
                continue;
            }
            const double z = (double)a[i] + (dt_bias ? (double)dt_bias[h] : 0.0);
            const double e = exp((double)A_log[h]);
            const double sig = 1.0 / (1.0 + exp(-z));
            const double g = -e * log1p(exp(z));
            da[i] = dg[i] * (-e * sig);
            const double beta = 1.0 / (1.0 + exp(-(double)b[i]));
            db[i] = dbeta[i] * beta * (1.0 - beta);
            if (dA_log)
                dA_log[h] += dg[i] * g;
            if (ddt_bias)
                ddt_bias[h] += da[i];
        }
    }
    return 0;
}

/*
 * Gradients of gdn_oracle_short_conv, in fp64, given dL/dy: with the window
 * x(s, c) (old state first, as in the forward), z[t] = bias + sum_j w[j] x(t-K+1+j)
 * and y = z sigmoid(z) (SiLU, derivative sigmoid(z) (1 + z (1 - sigmoid(z)))) or
 * y = z,
 *
 *   dz[t]        = dL/dy[t] * dy/dz
 *   dL/dx(s)    += w[j] dz[t]          for every t, j with s = t - K + 1 + j
 *   dL/dw[c][j]  = sum_t dz[t] x(t-K+1+j)
 *   dL/dbias[c]  = sum_t dz[t]
 *
 * over every sequence and token in order.  dL/dx for positions before the first
 * token is the gradient of the carried conv state (dstate, [N][C][K-1], oldest
 * first).  The state written after the sequence is a copy of inputs kept for the
 * next call, not a function the loss is taken of here.
 *
 * Inputs as gdn_oracle_short_conv plus dy [T][C] fp64.  Outputs, fp64: dx [T][C],
 * dw [C][K], dbias [C] (or NULL), dstate [N][C][K-1] (or NULL).
 */
int gdn_oracle_short_conv_backward(int32_t n_seqs, const int32_t *cu_seqlens, int32_t C, int32_t K,
                                   int32_t io_dtype, const void *x, const float *w, const float *bias,
                                   const double *state, int32_t silu, const double *dy,
                                   double *dx, double *dw, double *dbias, double *dstate)
{
    if (n_seqs < 0 || C <= 0 || K < 1 || (io_dtype != 0 && io_dtype != 1))
        return -1;
    if (!w || !dw)
        return -4;
    for (int64_t i = 0; i < (int64_t)C * K; ++i)
        dw[i] = 0.0;
    if (dbias)
        for (int32_t c = 0; c < C; ++c)
            dbias[c] = 0.0;
    if (n_seqs == 0)
        return 0;
    if (!cu_seqlens || (cu_seqlens[n_seqs] > 0 && (!x || !dy || !dx)))
        return -4;
    const int32_t M = K - 1;
    for (int32_t n = 0; n < n_seqs; ++n) {
        const int64_t tb = cu_seqlens[n], te = cu_seqlens[n + 1];
        if (te < tb)
            return -5;
        const int64_t len = te - tb;
        double *win = (double *)malloc(sizeof(double) * (size_t)(M + len + 1));
        double *dwin = (double *)malloc(sizeof(double) * (size_t)(M + len + 1));
        if (!win || !dwin) {
            free(win);
            free(dwin);
            return -6;
        }
        for (int32_t c = 0; c < C; ++c) {
            for (int32_t m = 0; m < M; ++m)
                win[m] = state ? state[((int64_t)n * C + c) * M + m] : 0.0;
            for (int64_t t = 0; t < len; ++t)
                win[M + t] = oracle_load(x, (tb + t) * C + c, io_dtype);
            for (int64_t s = 0; s < M + len; ++s)
                dwin[s] = 0.0;
            for (int64_t t = 0; t < len; ++t) {
                double z = bias ? (double)bias[c] : 0.0;
                for (int32_t j = 0; j < K; ++j)
                    z += (double)w[(int64_t)c * K + j] * win[t + j];
                double dz = dy[(tb + t) * C + c];
                if (silu) {
                    const double sig = 1.0 / (1.0 + exp(-z));
                    dz *= sig * (1.0 + z * (1.0 - sig));
                }
                for (int32_t j = 0; j < K; ++j) {
                    dwin[t + j] += (double)w[(int64_t)c * K + j] * dz;
                    dw[(int64_t)c * K + j] += dz * win[t + j];
                }
                if (dbias)
                    dbias[c] += dz;
            }
            for (int64_t t = 0; t < len; ++t)
                dx[(tb + t) * C + c] = dwin[M + t];
            if (dstate)
                for (int32_t m = 0; m < M; ++m)
                    dstate[((int64_t)n * C + c) * M + m] = dwin[m];
        }
        free(win);
        free(dwin);
    }
    return 0;
}

/*
 * Gradients of the recurrent forward (reverse-mode differentiation of the loop of
 * gdn_oracle_forward), in fp64.
 *
 * The page "Defending Against the Training-Inference Numeric Mismatch in RL
 * (Especially Linear Attention)" (section 3.2) keeps the training backward on the
 * chunked kernel while every forward runs the recurrence; forward parity says
 * nothing about gradients, so this function gives them from the definition.
 * Token t's forward step, exactly as gdn_oracle_forward takes it, is
 *
 *   Sd  = a S_{t-1}             (a = exp(g_t), b = beta_t)
 *   p   = Sd k                  (a dv-vector)
 *   u   = b (v - p)
 *   S_t = Sd + u k^T
 *   o   = S_t q
 *
 * and its adjoint, walked from the last token of a sequence to the first with
 * D = dL/dS_t (D = dhT, or 0, before the last token), is, line by line:
 *
 *   D  += dO q^T                 dq += S_t^T dO
 *   du  = D k                    dk += D^T u
 *   dv  = b du                   dbeta = du . (v - p)
 *   dp  = -b du
 *   Dd  = D + dp k^T             dk += Sd^T dp
 *   dg  = a <Dd, S_{t-1}>        (dL/da = <Dd, S_{t-1}>, da/dg = a)
 *   D   = a Dd                   (= dL/dS_{t-1})
 *
 * and dh0 = D after the first token.  dq and dk of key head kh add up over the
 * value heads that read it, in head order.
 *
 * The states S_{t-1} are not stored for the whole sequence: the forward pass keeps
 * one every ORACLE_CKPT tokens and the states of a stretch are recomputed from its
 * checkpoint by the same step, which gives the same values as keeping them all.
 *
 * Inputs as gdn_oracle_forward (dtype codes 0 fp32, 1 bf16 bits, 2 fp64), plus
 * dout [T][hv][dv] in dout_dtype and dhT [N][hv][dv][dk] fp64 or NULL (= 0).
 * Outputs, fp64: dq, dk [T][hk][dk]; dv [T][hv][dv]; dg, dbeta [T][hv];
 * dh0 [N][hv][dv][dk].
 */
#define ORACLE_CKPT 32

/* One forward step on S (dv x dk, in place); p_out (dv) receives p = Sd k. */
static void oracle_step(double *S, int32_t dv, int32_t dk, double a, double b,
                        const double *kv, const double *vv, double *p_out)
{
    for (int64_t e = 0; e < (int64_t)dv * dk; ++e)
        S[e] = a * S[e];
    for (int32_t j = 0; j < dv; ++j) {
        double *row = S + (size_t)j * dk;
        double p = 0.0;
        for (int32_t i = 0; i < dk; ++i)
            p += row[i] * kv[i];
        const double u = b * (vv[j] - p);
        for (int32_t i = 0; i < dk; ++i)
            row[i] += u * kv[i];
        if (p_out)
            p_out[j] = p;
    }
}

int gdn_oracle_backward(int32_t n_seqs, const int32_t *cu_seqlens,
                        int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                        int32_t qk_dtype, int32_t v_dtype, int32_t gate_dtype, int32_t dout_dtype,
                        const void *q, const void *k, const void *v,
                        const void *g, const void *beta, const double *h0,
                        const void *dout, const double *dhT,
                        double *dq, double *dk_out, double *dv_out, double *dg, double *dbeta, double *dh0,
                        int32_t n_threads)
{
    if (n_seqs < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (hv % hk != 0)
        return -2;
    if (qk_dtype < 0 || qk_dtype > 2 || v_dtype < 0 || v_dtype > 2 || dout_dtype < 0 || dout_dtype > 2 ||
        (gate_dtype != 0 && gate_dtype != 2))
        return -3;
    if (n_seqs == 0)
        return 0;
    if (!cu_seqlens || !dh0)
        return -4;
    if (cu_seqlens[0] != 0)
        return -5;
    for (int32_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return -5;
    const int64_t total = cu_seqlens[n_seqs];
    if (total > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk_out || !dv_out || !dg || !dbeta))
        return -4;

    const int32_t group = hv / hk;
    const int64_t SZ = (int64_t)dv * dk;
    int status = 0;
    if (n_threads <= 0)
        n_threads = 1;
    if (total > 0) {
        memset(dq, 0, sizeof(double) * (size_t)total * hk * dk);
        memset(dk_out, 0, sizeof(double) * (size_t)total * hk * dk);
    }

    /* One unit = (sequence, key head): its value heads run in order, so the sums
       into dq and dk of that key head have a fixed order. */
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t unit = 0; unit < (int64_t)n_seqs * hk; ++unit) {
        const int32_t n = (int32_t)(unit / hk);
        const int32_t kh = (int32_t)(unit % hk);
        const int64_t tb = cu_seqlens[n], len = cu_seqlens[n + 1] - tb;
        const int64_t n_ck = len / ORACLE_CKPT + 1;
        double *ck = (double *)malloc(sizeof(double) * (size_t)(n_ck * SZ));
        double *st = (double *)malloc(sizeof(double) * (size_t)((ORACLE_CKPT + 1) * SZ));
        double *pv = (double *)malloc(sizeof(double) * (size_t)(ORACLE_CKPT * dv));
        double *D = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *kv = (double *)malloc(sizeof(double) * (size_t)dk);
        double *qv = (double *)malloc(sizeof(double) * (size_t)dk);
        double *vv = (double *)malloc(sizeof(double) * (size_t)dv);
        double *dO = (double *)malloc(sizeof(double) * (size_t)dv);
        double *du = (double *)malloc(sizeof(double) * (size_t)dv);
        double *dp = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!ck || !st || !pv || !D || !kv || !qv || !vv || !dO || !du || !dp) {
#pragma omp atomic write
            status = -6;
        } else {
            for (int32_t h = kh * group; h < (kh + 1) * group; ++h) {
                const size_t state_off = ((size_t)n * hv + h) * (size_t)SZ;
                /* forward pass, keeping the state before every ORACLE_CKPT-th token */
                double *S = st;
                for (int64_t e = 0; e < SZ; ++e)
                    S[e] = h0 ? h0[state_off + e] : 0.0;
                for (int64_t t = 0; t < len; ++t) {
                    if (t % ORACLE_CKPT == 0)
                        memcpy(ck + (t / ORACLE_CKPT) * SZ, S, sizeof(double) * (size_t)SZ);
                    const int64_t tt = tb + t;
                    for (int32_t i = 0; i < dk; ++i)
                        kv[i] = oracle_load(k, (tt * hk + kh) * (int64_t)dk + i, qk_dtype);
                    for (int32_t j = 0; j < dv; ++j)
                        vv[j] = oracle_load(v, (tt * hv + h) * (int64_t)dv + j, v_dtype);
                    oracle_step(S, dv, dk, exp(oracle_load(g, tt * hv + h, gate_dtype)),
                                oracle_load(beta, tt * hv + h, gate_dtype), kv, vv, NULL);
                }
                /* backward pass */
                for (int64_t e = 0; e < SZ; ++e)
                    D[e] = dhT ? dhT[state_off + e] : 0.0;
                for (int64_t c = (len - 1) / ORACLE_CKPT; len > 0 && c >= 0; --c) {
                    const int64_t c0 = c * ORACLE_CKPT;
                    const int64_t c1 = (c0 + ORACLE_CKPT < len) ? c0 + ORACLE_CKPT : len;
                    /* st[m] = state before token c0 + m, for m = 0 .. c1 - c0 */
                    memcpy(st, ck + c * SZ, sizeof(double) * (size_t)SZ);
                    for (int64_t t = c0; t < c1; ++t) {
                        const int64_t tt = tb + t, m = t - c0;
                        memcpy(st + (m + 1) * SZ, st + m * SZ, sizeof(double) * (size_t)SZ);
                        for (int32_t i = 0; i < dk; ++i)
                            kv[i] = oracle_load(k, (tt * hk + kh) * (int64_t)dk + i, qk_dtype);
                        for (int32_t j = 0; j < dv; ++j)
                            vv[j] = oracle_load(v, (tt * hv + h) * (int64_t)dv + j, v_dtype);
                        oracle_step(st + (m + 1) * SZ, dv, dk, exp(oracle_load(g, tt * hv + h, gate_dtype)),
                                    oracle_load(beta, tt * hv + h, gate_dtype), kv, vv, pv + m * dv);
                    }
                    for (int64_t t = c1 - 1; t >= c0; --t) {
                        const int64_t tt = tb + t, m = t - c0;
                        const double *Sprev = st + m * SZ, *Snew = st + (m + 1) * SZ, *p = pv + m * dv;
                        const double a = exp(oracle_load(g, tt * hv + h, gate_dtype));
                        const double b = oracle_load(beta, tt * hv + h, gate_dtype);
                        const int64_t qk_off = (tt * hk + kh) * (int64_t)dk, v_off = (tt * hv + h) * (int64_t)dv;
                        for (int32_t i = 0; i < dk; ++i) {
                            kv[i] = oracle_load(k, qk_off + i, qk_dtype);
                            qv[i] = oracle_load(q, qk_off + i, qk_dtype);
                        }
                        for (int32_t j = 0; j < dv; ++j) {
                            vv[j] = oracle_load(v, v_off + j, v_dtype);
                            dO[j] = oracle_load(dout, v_off + j, dout_dtype);
                        }
                        /* o = S_t q */
                        for (int32_t j = 0; j < dv; ++j)
                            for (int32_t i = 0; i < dk; ++i) {
                                D[(size_t)j * dk + i] += dO[j] * qv[i];
                                dq[qk_off + i] += Snew[(size_t)j * dk + i] * dO[j];
                            }
                        /* S_t = Sd + u k^T, u = b (v - p) */
                        double db = 0.0;
                        for (int32_t j = 0; j < dv; ++j) {
                            double s = 0.0;
                            for (int32_t i = 0; i < dk; ++i)
                                s += D[(size_t)j * dk + i] * kv[i];
                            du[j] = s;
                            const double u = b * (vv[j] - p[j]);
                            for (int32_t i = 0; i < dk; ++i)
                                dk_out[qk_off + i] += D[(size_t)j * dk + i] * u;
                            dv_out[v_off + j] = b * du[j];
                            db += du[j] * (vv[j] - p[j]);
                            dp[j] = -b * du[j];
                        }
                        dbeta[tt * hv + h] = db;
                        /* p = Sd k, Sd = a S_{t-1} */
                        double da = 0.0;
                        for (int32_t j = 0; j < dv; ++j)
                            for (int32_t i = 0; i < dk; ++i) {
                                const size_t e = (size_t)j * dk + i;
                                D[e] += dp[j] * kv[i];
                                dk_out[qk_off + i] += a * Sprev[e] * dp[j];
                                da += D[e] * Sprev[e];
                                D[e] = a * D[e];
                            }
                        dg[tt * hv + h] = a * da;
                    }
                }
                memcpy(dh0 + state_off, D, sizeof(double) * (size_t)SZ);
            }
        }
        free(ck); free(st); free(pv); free(D); free(kv); free(qv); free(vv); free(dO); free(du); free(dp);
    }
    return status;
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
