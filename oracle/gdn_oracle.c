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
 *   q, k   : [T][hk][dk]   fp32 (io_dtype 0) or bf16 bits (io_dtype 1)
 *   v      : [T][hv][dv]   same dtype as q
 *   g, beta: [T][hv]       fp32
 *   h0, hT : [N][hv][dv][dk] fp64 (h0 may be NULL = zero state, hT may be NULL)
 *   out    : [T][hv][dv]   fp64
 *   cu_seqlens: [N+1] int32, cu[0] = 0, non-decreasing, cu[N] = T.
 *
 * Parallelism: OpenMP over independent (sequence, value head) units only; the
 * arithmetic inside a unit is the sequential loop above.
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
    /* bf16 is the top half of an IEEE binary32; the widening is exact. */
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Returns 0 on success, a negative value on a bad argument. */
int gdn_oracle_forward(int32_t n_seqs, const int32_t *cu_seqlens,
                       int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                       int32_t io_dtype,
                       const void *q, const void *k, const void *v,
                       const float *g, const float *beta,
                       const double *h0, double *out, double *hT,
                       int32_t n_threads)
{
    if (n_seqs < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (hv % hk != 0)
        return -2;
    if (io_dtype != 0 && io_dtype != 1)
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
            const double a = exp((double)g[t * hv + h]);
            const double b = (double)beta[t * hv + h];
            const int64_t qk_off = (t * hk + kh) * (int64_t)dk;
            const int64_t v_off = (t * hv + h) * (int64_t)dv;

            for (int64_t e = 0; e < (int64_t)dv * dk; ++e)
                S[e] = a * S[e];

            for (int32_t j = 0; j < dv; ++j) {
                double *row = S + (size_t)j * dk;
                double p = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    p += row[i] * oracle_load(k, qk_off + i, io_dtype);
                const double u = b * (oracle_load(v, v_off + j, io_dtype) - p);
                for (int32_t i = 0; i < dk; ++i)
                    row[i] += u * oracle_load(k, qk_off + i, io_dtype);
                double o = 0.0;
                for (int32_t i = 0; i < dk; ++i)
                    o += row[i] * oracle_load(q, qk_off + i, io_dtype);
                out[v_off + j] = o;
            }
        }
        if (hT)
            memcpy(hT + state_off, S, sizeof(double) * (size_t)dv * (size_t)dk);
        free(S);
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
