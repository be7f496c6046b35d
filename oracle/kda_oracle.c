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

/*
 * Backward pass (reverse-mode derivative) of the same recurrence, fp64 --
 * TEST INFRASTRUCTURE ONLY.
 *
 * Given the gradients dO of every o_t and dS_T of the final states (NULL =
 * zeros), returns the gradients of q, k, v, beta, g (= log alpha) and S0.
 * Per sequence and head, with G the gradient of the loss with respect to
 * the state after token t, the steps of the forward pass are undone in
 * reverse order (write, delta, probe, decay):
 *
 *   G     += q_t do_t^T                         read-out o_t = S_t^T q_t
 *   dq_t   = S_t do_t
 *   P      = Diag(alpha_t) S_{t-1}              the decayed state
 *   e      = v_t - P^T k_t                      the delta
 *   de     = beta_t G^T k_t                     S_t = P + beta_t k_t e^T
 *   dv_t   = de                                 e = v_t - P^T k_t
 *   dbeta_t = k_t^T G e
 *   dk_t   = beta_t G e - P de
 *   dP     = G - k_t de^T
 *   dg_t   = alpha_t * rowsum(dP * S_{t-1})     P = Diag(exp(g_t)) S_{t-1}
 *   G      = Diag(alpha_t) dP                   (gradient of S_{t-1})
 *
 * and dS0 is G after the first token.  The states S_{t-1} are recomputed
 * block by block from states stored every BLK tokens in a forward sweep.
 * Work is split over (sequence, head) only: dq, dk, dbeta, dg sum over all
 * value columns.
 */
#define BLK 64

int kda_oracle_backward(int64_t total_tokens, int32_t n_seqs, int32_t n_heads,
                        int32_t d_k, int32_t d_v,
                        const double* q, const double* k, const double* v,
                        const double* beta, const double* g,
                        const double* S0, const int64_t* cu_seqlens,
                        const double* dO, const double* dS_T,
                        double* dq, double* dk, double* dv, double* dbeta,
                        double* dg, double* dS0, int n_threads)
{
    if (n_seqs <= 0 || n_heads <= 0 || d_k <= 0 || d_v <= 0 || !cu_seqlens || !dO) return 1;
    if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != total_tokens) return 2;
    for (int32_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return 2;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    const int64_t SS = (int64_t)d_k * d_v;
    const int64_t n_tasks = (int64_t)n_seqs * n_heads;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t task = 0; task < n_tasks; ++task) {
        const int64_t h = task % n_heads, n = task / n_heads;
        const int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1], L = t1 - t0;
        const int64_t n_blk = (L + BLK - 1) / BLK;
        /* ckpt[b] = state before token t0 + b*BLK; blk[i] = state after token i of the current block */
        double* ckpt = (double*)malloc((size_t)((n_blk > 0 ? n_blk : 1) * SS) * sizeof(double));
        double* blk = (double*)malloc((size_t)((BLK + 1) * SS) * sizeof(double));
        double* G = (double*)malloc((size_t)SS * sizeof(double));
        double* Pm = (double*)malloc((size_t)SS * sizeof(double));
        double* alpha = (double*)malloc((size_t)d_k * sizeof(double));
        double* e = (double*)malloc((size_t)d_v * sizeof(double));
        double* de = (double*)malloc((size_t)d_v * sizeof(double));
        if (!ckpt || !blk || !G || !Pm || !alpha || !e || !de) {
            free(ckpt); free(blk); free(G); free(Pm); free(alpha); free(e); free(de);
            bad = 1;
            continue;
        }
        const double* s0 = S0 ? S0 + (n * n_heads + h) * SS : NULL;
        /* one token of the forward recurrence: S (in) -> S (out), in place */
        #define KDA_STEP(Sx, t)                                                        \
            do {                                                                        \
                const double* kt_ = k + ((t) * n_heads + h) * d_k;                      \
                const double* vt_ = v + ((t) * n_heads + h) * d_v;                      \
                const double* gt_ = g + ((t) * n_heads + h) * d_k;                      \
                const double bt_ = beta[(t) * n_heads + h];                             \
                for (int64_t i = 0; i < d_k; ++i)                                       \
                    for (int64_t j = 0; j < d_v; ++j) (Sx)[i * d_v + j] *= exp(gt_[i]); \
                for (int64_t j = 0; j < d_v; ++j) {                                     \
                    double p_ = 0.0;                                                    \
                    for (int64_t i = 0; i < d_k; ++i) p_ += (Sx)[i * d_v + j] * kt_[i]; \
                    e[j] = vt_[j] - p_;                                                 \
                }                                                                       \
                for (int64_t i = 0; i < d_k; ++i)                                       \
                    for (int64_t j = 0; j < d_v; ++j) (Sx)[i * d_v + j] += bt_ * kt_[i] * e[j]; \
            } while (0)

        /* forward sweep: checkpoints */
        for (int64_t i = 0; i < SS; ++i) G[i] = s0 ? s0[i] : 0.0;   /* G used as the running state here */
        for (int64_t b = 0; b < n_blk; ++b) {
            memcpy(ckpt + b * SS, G, (size_t)SS * sizeof(double));
            const int64_t te = (t0 + (b + 1) * BLK < t1) ? t0 + (b + 1) * BLK : t1;
            for (int64_t t = t0 + b * BLK; t < te; ++t) KDA_STEP(G, t);
        }
        /* backward sweep */
        for (int64_t i = 0; i < SS; ++i) G[i] = dS_T ? dS_T[(n * n_heads + h) * SS + i] : 0.0;
        for (int64_t b = n_blk - 1; b >= 0; --b) {
            const int64_t tb = t0 + b * BLK;
            const int64_t te = (tb + BLK < t1) ? tb + BLK : t1;
            memcpy(blk, ckpt + b * SS, (size_t)SS * sizeof(double));
            for (int64_t t = tb; t < te; ++t) {
                memcpy(blk + (t - tb + 1) * SS, blk + (t - tb) * SS, (size_t)SS * sizeof(double));
                KDA_STEP(blk + (t - tb + 1) * SS, t);
            }
            for (int64_t t = te - 1; t >= tb; --t) {
                const double* Sprev = blk + (t - tb) * SS;     /* S_{t-1} */
                const double* Scur = blk + (t - tb + 1) * SS;  /* S_t */
                const double* qt = q + (t * n_heads + h) * d_k;
                const double* kt = k + (t * n_heads + h) * d_k;
                const double* vt = v + (t * n_heads + h) * d_v;
                const double* gt = g + (t * n_heads + h) * d_k;
                const double* dot = dO + (t * n_heads + h) * d_v;
                const double bt = beta[t * n_heads + h];
                /* read-out */
                for (int64_t i = 0; i < d_k; ++i)
                    for (int64_t j = 0; j < d_v; ++j) G[i * d_v + j] += qt[i] * dot[j];
                for (int64_t i = 0; i < d_k; ++i) {
                    double s = 0.0;
                    for (int64_t j = 0; j < d_v; ++j) s += Scur[i * d_v + j] * dot[j];
                    dq[(t * n_heads + h) * d_k + i] = s;
                }
                /* decayed state and delta */
                for (int64_t i = 0; i < d_k; ++i) {
                    alpha[i] = exp(gt[i]);
                    for (int64_t j = 0; j < d_v; ++j) Pm[i * d_v + j] = alpha[i] * Sprev[i * d_v + j];
                }
                for (int64_t j = 0; j < d_v; ++j) {
                    double p = 0.0, gk = 0.0;
                    for (int64_t i = 0; i < d_k; ++i) {
                        p += Pm[i * d_v + j] * kt[i];
                        gk += G[i * d_v + j] * kt[i];
                    }
                    e[j] = vt[j] - p;
                    de[j] = bt * gk;
                    dv[(t * n_heads + h) * d_v + j] = de[j];
                }
                double db = 0.0;
                for (int64_t i = 0; i < d_k; ++i) {
                    double ge = 0.0, pde = 0.0;
                    for (int64_t j = 0; j < d_v; ++j) {
                        ge += G[i * d_v + j] * e[j];
                        pde += Pm[i * d_v + j] * de[j];
                    }
                    db += kt[i] * ge;
                    dk[(t * n_heads + h) * d_k + i] = bt * ge - pde;
                }
                dbeta[t * n_heads + h] = db;
                /* dP = G - k de^T; dg; G <- Diag(alpha) dP */
                for (int64_t i = 0; i < d_k; ++i) {
                    double s = 0.0;
                    for (int64_t j = 0; j < d_v; ++j) {
                        const double dp = G[i * d_v + j] - kt[i] * de[j];
                        s += dp * Sprev[i * d_v + j];
                        G[i * d_v + j] = alpha[i] * dp;
                    }
                    dg[(t * n_heads + h) * d_k + i] = alpha[i] * s;
                }
            }
        }
        if (dS0)
            for (int64_t i = 0; i < SS; ++i) dS0[(n * n_heads + h) * SS + i] = G[i];
        #undef KDA_STEP
        free(ckpt); free(blk); free(G); free(Pm); free(alpha); free(e); free(de);
    }
    return bad ? 4 : 0;
}
