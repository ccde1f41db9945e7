/*
 * CPU oracle for the gated delta rule.  TEST INFRASTRUCTURE ONLY: nothing on
 * the product path may link, load or call this file.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark use it.
 *
 * What it computes (fp64 throughout, token by token, no chunking):
 *
 *   The recurrence of the research-map summary "Gated Delta Networks:
 *   Improving Mamba2 with Delta Rule", section "Approach", restated in the
 *   blog "Gated DeltaNet: Harmonizing Gating and the Delta Rule for Superior
 *   Linear RNNs", section "Methodology: The Gated Delta Rule":
 *
 *       S_t = S_{t-1} ( alpha_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T
 *
 *   with S_t a d_v x d_k matrix (the write v k^T is d_v x d_k).  Multiplying
 *   out the bracket gives the identical rank-one form used below:
 *
 *       p   = S_{t-1} k_t                       (the current read)
 *       S_t = alpha_t S_{t-1} + (beta_t v_t - alpha_t beta_t p) k_t^T
 *
 *   The pages write no output equation; the read-out used here is the
 *   post-update read o_t = S_t q_t, with no scale on q.
 *
 *   The gate is passed as log(alpha_t) and exponentiated here, once per token.
 *
 * Layouts (row-major, the same arrays the GPU library receives, upcast to
 * double): q,k [B,T,H,d_k]; v,o [B,T,H,d_v]; log_alpha, beta [B,T,H];
 * S0, S_T [units,H,d_v,d_k] where units = B, or n_seqs when cu_seqlens packs
 * several sequences into one row of T tokens (then B must be 1).
 *
 * Parity unpinned by the pages themselves: they print no worked example.
 * The tests pin this code to closed forms instead (scalar decay at beta=0,
 * DeltaNet at alpha=1, exact writes on orthonormal keys, the explicit
 * product form on tiny inputs, the per-step regression identity).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (sequence, head) unit over L tokens.  ts_k / ts_v are the strides, in
 * elements, between consecutive tokens of q,k and of v,o; ts_g the stride of
 * the per-token gate arrays. */
static void run_unit(long L, int dk, int dv,
                     const double *q, const double *k, const double *v,
                     const double *log_alpha, const double *beta,
                     long ts_k, long ts_v, long ts_g,
                     const double *S0, double *o, double *S_T,
                     double *S, double *p)
{
    for (long e = 0; e < (long)dv * dk; ++e) S[e] = S0 ? S0[e] : 0.0;

    for (long t = 0; t < L; ++t) {
        const double *kt = k + t * ts_k;
        const double *qt = q + t * ts_k;
        const double *vt = v + t * ts_v;
        const double a = exp(log_alpha[t * ts_g]);
        const double b = beta[t * ts_g];

        /* current read p = S k */
        for (int r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += S[(long)r * dk + c] * kt[c];
            p[r] = acc;
        }
        /* S <- a S + (b v - a b p) k^T */
        for (int r = 0; r < dv; ++r) {
            const double w = b * vt[r] - a * b * p[r];
            for (int c = 0; c < dk; ++c)
                S[(long)r * dk + c] = a * S[(long)r * dk + c] + w * kt[c];
        }
        /* o_t = S_t q_t (post-update state) */
        if (o) {
            double *ot = o + t * ts_v;
            for (int r = 0; r < dv; ++r) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += S[(long)r * dk + c] * qt[c];
                ot[r] = acc;
            }
        }
    }
    if (S_T)
        for (long e = 0; e < (long)dv * dk; ++e) S_T[e] = S[e];
}

/* Full forward over a batch (cu_seqlens == NULL or n_seqs == 0) or over
 * packed sequences.  Returns 0 on success, -1 on a bad argument or a failed
 * allocation.  o and S_T may be NULL (not written).  n_threads <= 0 lets
 * OpenMP choose. */
int gdn_oracle_fwd(int B, long T, int H, int dk, int dv,
                   int n_seqs, const int32_t *cu_seqlens,
                   const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta,
                   const double *S0, double *o, double *S_T, int n_threads)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !log_alpha || !beta) return -1;
    const int varlen = (cu_seqlens != NULL && n_seqs > 0);
    if (varlen && B != 1) return -1;
    const int units = varlen ? n_seqs : B;
    const long n_work = (long)units * H;
    int bad = 0;

#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long w = 0; w < n_work; ++w) {
        const int u = (int)(w / H), h = (int)(w % H);
        long t0, L;
        if (varlen) {
            t0 = cu_seqlens[u];
            L = (long)cu_seqlens[u + 1] - cu_seqlens[u];
            if (t0 < 0 || L < 0 || t0 + L > T) { bad |= 1; continue; }
        } else {
            t0 = (long)u * T;
            L = T;
        }
        double *S = (double *)malloc(sizeof(double) * ((size_t)dv * dk + dv));
        if (!S) { bad |= 1; continue; }
        const long gk = t0 * H + h;                 /* token-head row index */
        const long unit_state = ((long)u * H + h) * dv * dk;
        run_unit(L, dk, dv,
                 q + gk * dk, k + gk * dk, v + gk * dv,
                 log_alpha + gk, beta + gk,
                 (long)H * dk, (long)H * dv, H,
                 S0 ? S0 + unit_state : NULL,
                 o ? o + gk * dv : NULL,
                 S_T ? S_T + unit_state : NULL,
                 S, S + (size_t)dv * dk);
        free(S);
    }
    return bad ? -1 : 0;
}

/* One recurrent decode step for every (b,h): the same body with one token,
 * the state S [B,H,d_v,d_k] updated in place.  q,k [B,H,d_k]; v,o [B,H,d_v];
 * log_alpha, beta [B,H]. */
int gdn_oracle_step(int B, int H, int dk, int dv,
                    const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *beta,
                    double *S, double *o, int n_threads)
{
    if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !log_alpha || !beta || !S) return -1;
    /* A [B,H,...] step is a forward over T=1 with the token axis of length 1,
     * which has the same memory layout. */
    return gdn_oracle_fwd(B, 1, H, dk, dv, 0, NULL, q, k, v, log_alpha, beta,
                          S, o, S, n_threads);
}
