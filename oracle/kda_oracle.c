/*
 * KDA forward oracle: the token-by-token recurrence in fp64, plain C.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library. It shares no code
 * with the HIP path and nothing here is tuned for speed beyond running
 * independent (sequence, head) chains on OpenMP threads.
 *
 * What it computes (FlashInfer "kda_backward" page, "Supported contract";
 * the Trainium kda-neuron-kernels commit log, the per-K decay fix T-KDA-02):
 *
 *   for every sequence n (tokens cu[n] .. cu[n+1]-1) and head h:
 *     S[V][K] = h0[n,h] or 0                  value-first state, fp64
 *     for each token t:
 *       qh = q_t / sqrt(sum q_t^2 + eps) * scale
 *       kh = k_t / sqrt(sum k_t^2 + eps)
 *       lambda_c = lb * sigmoid(exp(A_log[h]) * (g_t[c] + dt_bias[h,c]))
 *       alpha_c  = exp(lambda_c)              decay per KEY channel
 *       b        = sigmoid(beta_raw_t)
 *       S[:,c]  *= alpha_c                    (columns of the [V,K] state)
 *       p        = S kh                       prediction from the decayed state
 *       S       += b (v_t - p) kh^T           delta-rule write
 *       o_t      = S qh                       read after the write
 *     ht[n,h] = S
 *
 * Readings where the pages are silent: eps is added inside the square root;
 * the scale is folded into qh; the decay is applied before the prediction and
 * the output is read after the write (the order in which the contract lists
 * decay, update and read-out). Inputs are passed as fp32 (bf16 values upcast
 * exactly) and converted to fp64 element by element; the initial and final
 * states are fp64 so that runs can be chained without rounding.
 *
 * Parity pins: T=1 closed form, beta=0 pure decay, orthonormal-key
 * write/recall, constant-key moving average, varlen and split invariance,
 * linearity, the K=V=1 scalar recurrence and agreement with the independent
 * chunked form in chunked.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Logistic function evaluated without overflow for any finite x. */
static double sigmoid(double x)
{
    if (x >= 0.0) {
        double z = exp(-x);
        return 1.0 / (1.0 + z);
    } else {
        double z = exp(x);
        return z / (1.0 + z);
    }
}

/* Returns 0 on success, a negative number for invalid arguments, -100 when
 * out of host memory. Layouts (row-major, token-major, packed along T):
 *   q, k, g : [T, H, K] fp32     v : [T, H, V] fp32     beta_raw : [T, H]
 *   A_log   : [H]                dt_bias : [H, K]
 *   cu      : [N+1] int64, cu[0] = 0, non-decreasing, cu[N] = T
 *   h0      : [N, H, V, K] fp64 or NULL (zero initial state)
 *   o       : [T, H, V] fp64 (written)     ht : [N, H, V, K] fp64 or NULL
 */
int oracle_kda_recurrent(const float *q, const float *k, const float *v,
                         const float *g, const float *beta_raw,
                         const float *A_log, const float *dt_bias,
                         double scale, double lower_bound, double eps,
                         const int64_t *cu, int64_t N, int64_t H,
                         int64_t K, int64_t V,
                         const double *h0, double *o, double *ht,
                         int nthreads)
{
    if (!q || !k || !v || !g || !beta_raw || !A_log || !dt_bias || !cu || !o)
        return -1;
    if (N < 0 || H < 1 || K < 1 || V < 1)
        return -2;
    for (int64_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n] || cu[0] != 0)
            return -3;

    int bad = 0;
    int64_t chains = N * H;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : bad)
#endif
    for (int64_t idx = 0; idx < chains; ++idx) {
        int64_t n = idx / H, h = idx % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(V * K));
        double *qh = (double *)malloc(sizeof(double) * (size_t)K);
        double *kh = (double *)malloc(sizeof(double) * (size_t)K);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)K);
        double *p = (double *)malloc(sizeof(double) * (size_t)V);
        if (!S || !qh || !kh || !alpha || !p) {
            free(S); free(qh); free(kh); free(alpha); free(p);
            bad |= 1;
            continue;
        }
        const double *S0 = h0 ? h0 + idx * V * K : NULL;
        for (int64_t i = 0; i < V * K; ++i)
            S[i] = S0 ? S0[i] : 0.0;
        double a = exp((double)A_log[h]);

        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const float *qt = q + (t * H + h) * K;
            const float *kt = k + (t * H + h) * K;
            const float *vt = v + (t * H + h) * V;
            const float *gt = g + (t * H + h) * K;

            /* L2 normalisation of q and k; the output scale rides on q. */
            double sq = 0.0, sk = 0.0;
            for (int64_t c = 0; c < K; ++c) {
                sq += (double)qt[c] * (double)qt[c];
                sk += (double)kt[c] * (double)kt[c];
            }
            double rq = 1.0 / sqrt(sq + eps), rk = 1.0 / sqrt(sk + eps);
            for (int64_t c = 0; c < K; ++c) {
                qh[c] = (double)qt[c] * rq * scale;
                kh[c] = (double)kt[c] * rk;
            }

            /* Gate: per-key-channel log-decay lambda in (lb, 0), alpha = e^lambda. */
            for (int64_t c = 0; c < K; ++c) {
                double x = a * ((double)gt[c] + (double)dt_bias[h * K + c]);
                alpha[c] = exp(lower_bound * sigmoid(x));
            }
            double b = sigmoid((double)beta_raw[t * H + h]);

            /* 1. decay every key channel (column c of the value-first state) */
            for (int64_t r = 0; r < V; ++r)
                for (int64_t c = 0; c < K; ++c)
                    S[r * K + c] *= alpha[c];
            /* 2. prediction p = S kh from the decayed state */
            for (int64_t r = 0; r < V; ++r) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c)
                    acc += S[r * K + c] * kh[c];
                p[r] = acc;
            }
            /* 3. delta-rule write S += b (v - p) kh^T */
            for (int64_t r = 0; r < V; ++r) {
                double u = b * ((double)vt[r] - p[r]);
                for (int64_t c = 0; c < K; ++c)
                    S[r * K + c] += u * kh[c];
            }
            /* 4. read-out after the write: o = S qh */
            double *ot = o + (t * H + h) * V;
            for (int64_t r = 0; r < V; ++r) {
                double acc = 0.0;
                for (int64_t c = 0; c < K; ++c)
                    acc += S[r * K + c] * qh[c];
                ot[r] = acc;
            }
        }
        if (ht)
            memcpy(ht + idx * V * K, S, sizeof(double) * (size_t)(V * K));
        free(S); free(qh); free(kh); free(alpha); free(p);
    }
    return bad ? -100 : 0;
}

/* Number of OpenMP threads a call with nthreads <= 0 would use. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
