/*
 * Plain fp64 CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this.  It shares no code, header or table with the GPU library.
 *
 * What it computes (per sequence n and head h, from S = S0[n,h], or zeros):
 *
 *   for each token t of the sequence, in order:
 *     S-   = Diag(alpha_t) S              alpha_t = exp(g_t), per key channel
 *     vhat = S-^T k_t                     probe the memory with the key
 *     e    = v_t - vhat                   the delta (wanted minus returned)
 *     S    = S- + beta_t k_t e^T          write the delta with strength beta
 *     o_t  = S^T q_t                      read-out after the write
 *   S_T = S
 *
 * This is the per-head state recurrence and its delta-rule decomposition of
 * the ogis-ri NLP primer on Kimi K3, §3.1 "KDA（Kimi Delta Attention）"
 * (decay, probe, error, write; S is d_k x d_v, q/k are d_k, v is d_v,
 * alpha is a per-channel d_k vector, beta a scalar; read-out o_t = S_t^T q_t).
 * The read-out uses the state after the token's own write: the pages' chunk
 * form keeps the diagonal (i <= j) in the intra-chunk term.
 *
 * No scale, normalisation or clamp is applied: inputs are used as given.
 * Columns of S evolve independently (every operator acts from the left), so
 * the work is split over (sequence, head, block of value columns).
 *
 * Layout: q, k, g [T_total, H, d_k]; v [T_total, H, d_v]; beta [T_total, H];
 * S0, S_T [N, H, d_k, d_v]; o [(out_hi - out_lo), H, d_v] for packed tokens in
 * [out_lo, out_hi).  cu_seqlens [N+1] on the host.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define COLS 16

int kda_oracle_forward(int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                       int32_t d_k, int32_t d_v,
                       const double* q, const double* k, const double* v,
                       const double* beta, const double* g,
                       const double* S0, const int64_t* cu_seqlens,
                       int64_t out_lo, int64_t out_hi, double* o,
                       double* S_T, int n_threads)
{
    if (n_seqs <= 0 || n_heads <= 0 || d_k <= 0 || d_v <= 0 || !cu_seqlens) return 1;
    if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != total_tokens) return 2;
    for (int32_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
    if (out_hi < out_lo) return 3;

    const int64_t n_cb = (d_v + COLS - 1) / COLS;
    const int64_t n_tasks = (int64_t)n_seqs * n_heads * n_cb;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
        const int64_t cb = task % n_cb;
        const int64_t h = (task / n_cb) % n_heads;
        const int64_t n = task / (n_cb * n_heads);
        const int64_t c0 = cb * COLS;
        const int64_t nc = (d_v - c0 < COLS) ? (d_v - c0) : COLS;

        double* S = (double*)calloc((size_t)d_k * COLS, sizeof(double));
        double* alpha = (double*)malloc((size_t)d_k * sizeof(double));
        if (!S || !alpha) { free(S); free(alpha); bad = 1; continue; }
        if (S0)
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < nc; ++j)
                    S[i * COLS + j] = S0[((n * n_heads + h) * d_k + i) * d_v + c0 + j];

        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const double* qt = q + (t * n_heads + h) * d_k;
            const double* kt = k + (t * n_heads + h) * d_k;
            const double* vt = v + (t * n_heads + h) * d_v + c0;
            const double* gt = g + (t * n_heads + h) * d_k;
            const double bt = beta[t * n_heads + h];
            double vhat[COLS], e[COLS];

            /* decay: S- = Diag(exp(g_t)) S */
            for (int64_t i = 0; i < d_k; ++i) alpha[i] = exp(gt[i]);
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < nc; ++j) S[i * COLS + j] *= alpha[i];
            /* probe: vhat = S-^T k_t */
            for (int64_t j = 0; j < nc; ++j) vhat[j] = 0.0;
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < nc; ++j) vhat[j] += S[i * COLS + j] * kt[i];
            /* delta: e = v_t - vhat */
            for (int64_t j = 0; j < nc; ++j) e[j] = vt[j] - vhat[j];
            /* write: S = S- + beta_t k_t e^T */
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < nc; ++j) S[i * COLS + j] += bt * kt[i] * e[j];
            /* read-out: o_t = S^T q_t */
            if (o && t >= out_lo && t < out_hi) {
                double* ot = o + ((t - out_lo) * n_heads + h) * d_v + c0;
                for (int64_t j = 0; j < nc; ++j) ot[j] = 0.0;
                for (int64_t i = 0; i < d_k; ++i)
                    for (int64_t j = 0; j < nc; ++j) ot[j] += S[i * COLS + j] * qt[i];
            }
        }
        if (S_T)
            for (int64_t i = 0; i < d_k; ++i)
                for (int64_t j = 0; j < nc; ++j)
                    S_T[((n * n_heads + h) * d_k + i) * d_v + c0 + j] = S[i * COLS + j];
        free(S);
        free(alpha);
    }
    return bad ? 4 : 0;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
