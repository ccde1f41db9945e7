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

/* ------------------------------------------------------------------------
 * Backward pass (reverse mode of the recurrence above), fp64.
 *
 * The pages name a backward pass as part of efficient parallel training
 * ("Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention",
 * abstract: a gate-aware backward pass; blog "Gated DeltaNet: Harmonizing
 * Gating and the Delta Rule for Superior Linear RNNs", section
 * "Hardware-Efficient Training") but print none; a backward pass is fixed by
 * its forward: the gradient of L = sum_t <dO_t, o_t> + <dS_T, S_T> with
 * respect to every input.  Written here as the chain rule through each token
 * in reverse order, for the step
 *
 *     p = S_{t-1} k,  u = beta (v - alpha p),  S_t = alpha S_{t-1} + u k^T,
 *     o_t = S_t q,    alpha = e^{log_alpha}.
 *
 * With G the gradient of L with respect to S_t (dS_T after the last token):
 *     G   += dO_t q^T                  (o_t reads the post-update state)
 *     dq   = S_t^T dO_t
 *     du   = G k,       dk = G^T u + S_{t-1}^T dp,   dp = -alpha beta du
 *     dv   = beta du,   dbeta = du . (v - alpha p)
 *     dalpha = <G, S_{t-1}> - beta du . p,           dlog_alpha = alpha dalpha
 *     G_{t-1} = alpha G + dp k^T
 * and dS0 = G_0.  The states S_{t-1} are recomputed forward from
 * checkpoints taken every kSeg tokens, one segment at a time.
 * ------------------------------------------------------------------------ */
enum { kSeg = 32 };

static void bwd_unit(long L, int dk, int dv,
                     const double *q, const double *k, const double *v,
                     const double *log_alpha, const double *beta,
                     long ts_k, long ts_v, long ts_g,
                     const double *S0, const double *dO, const double *dS_T,
                     double *dq, double *dk_out, double *dv_out,
                     double *dla, double *dbeta, double *dS0,
                     double *ck, double *seg, double *G, double *p, double *du, double *dp)
{
    const long n = (long)dv * dk;
    const long nck = (L + kSeg - 1) / kSeg;
    /* forward: checkpoint j holds the state before token j * kSeg */
    double *run = seg;   /* scratch for the running state */
    for (long e = 0; e < n; ++e) run[e] = (S0 != NULL) ? S0[e] : 0.0;
    for (long t = 0; t < L; ++t) {
        if (t % kSeg == 0) memcpy(ck + (t / kSeg) * n, run, sizeof(double) * n);
        const double *kt = k + t * ts_k, *vt = v + t * ts_v;
        const double a = exp(log_alpha[t * ts_g]), b = beta[t * ts_g];
        for (int r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += run[(long)r * dk + c] * kt[c];
            const double w = b * vt[r] - a * b * acc;
            for (int c = 0; c < dk; ++c)
                run[(long)r * dk + c] = a * run[(long)r * dk + c] + w * kt[c];
        }
    }
    for (long e = 0; e < n; ++e) G[e] = dS_T ? dS_T[e] : 0.0;

    for (long j = nck - 1; j >= 0; --j) {
        const long t0 = j * kSeg, t1 = (t0 + kSeg < L) ? t0 + kSeg : L;
        /* seg[i] = state after token t0 + i - 1, i.e. seg[0] = checkpoint */
        memcpy(seg, ck + j * n, sizeof(double) * n);
        for (long t = t0; t < t1; ++t) {
            const double *Sp = seg + (t - t0) * n;
            double *Sn = seg + (t - t0 + 1) * n;
            const double *kt = k + t * ts_k, *vt = v + t * ts_v;
            const double a = exp(log_alpha[t * ts_g]), b = beta[t * ts_g];
            for (int r = 0; r < dv; ++r) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += Sp[(long)r * dk + c] * kt[c];
                const double w = b * vt[r] - a * b * acc;
                for (int c = 0; c < dk; ++c)
                    Sn[(long)r * dk + c] = a * Sp[(long)r * dk + c] + w * kt[c];
            }
        }
        for (long t = t1 - 1; t >= t0; --t) {
            const double *Sp = seg + (t - t0) * n;       /* S_{t-1} */
            const double *Sn = seg + (t - t0 + 1) * n;   /* S_t */
            const double *kt = k + t * ts_k, *qt = q + t * ts_k, *vt = v + t * ts_v;
            const double *dot = dO + t * ts_v;
            const double a = exp(log_alpha[t * ts_g]), b = beta[t * ts_g];
            double *dqt = dq + t * ts_k, *dkt = dk_out + t * ts_k, *dvt = dv_out + t * ts_v;
            /* G += dO_t q^T */
            for (int r = 0; r < dv; ++r)
                for (int c = 0; c < dk; ++c) G[(long)r * dk + c] += dot[r] * qt[c];
            /* dq = S_t^T dO_t */
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int r = 0; r < dv; ++r) acc += Sn[(long)r * dk + c] * dot[r];
                dqt[c] = acc;
            }
            /* p = S_{t-1} k, du = G k */
            for (int r = 0; r < dv; ++r) {
                double ap = 0.0, ag = 0.0;
                for (int c = 0; c < dk; ++c) {
                    ap += Sp[(long)r * dk + c] * kt[c];
                    ag += G[(long)r * dk + c] * kt[c];
                }
                p[r] = ap;
                du[r] = ag;
            }
            double db = 0.0, dup = 0.0;
            for (int r = 0; r < dv; ++r) {
                db += du[r] * (vt[r] - a * p[r]);
                dup += du[r] * p[r];
                dvt[r] = b * du[r];
                dp[r] = -a * b * du[r];
            }
            /* dk = G^T u + S_{t-1}^T dp, with u = beta (v - alpha p) */
            for (int c = 0; c < dk; ++c) {
                double acc = 0.0;
                for (int r = 0; r < dv; ++r)
                    acc += G[(long)r * dk + c] * b * (vt[r] - a * p[r]) + Sp[(long)r * dk + c] * dp[r];
                dkt[c] = acc;
            }
            /* dalpha = <G, S_{t-1}> - beta du . p */
            double gs = 0.0;
            for (long e = 0; e < n; ++e) gs += G[e] * Sp[e];
            dla[t * ts_g] = a * (gs - b * dup);
            dbeta[t * ts_g] = db;
            /* G_{t-1} = alpha G + dp k^T */
            for (int r = 0; r < dv; ++r)
                for (int c = 0; c < dk; ++c)
                    G[(long)r * dk + c] = a * G[(long)r * dk + c] + dp[r] * kt[c];
        }
    }
    if (dS0)
        for (long e = 0; e < n; ++e) dS0[e] = G[e];
}

/* Gradients of L = sum <dO, o> + <dS_T, S_T> for the forward of
 * gdn_oracle_fwd (same layouts; dS_T may be NULL = zero).  Outputs dq, dk
 * [B,T,H,d_k]; dv [B,T,H,d_v]; dlog_alpha, dbeta [B,T,H]; dS0 [units,H,d_v,d_k]
 * (may be NULL).  Returns 0 on success, -1 on a bad argument or allocation. */
int gdn_oracle_bwd(int B, long T, int H, int dk, int dv,
                   int n_seqs, const int32_t *cu_seqlens,
                   const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta, const double *S0,
                   const double *dO, const double *dS_T,
                   double *dq, double *dk_out, double *dv_out,
                   double *dlog_alpha, double *dbeta, double *dS0, int n_threads)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !log_alpha || !beta || !dO) return -1;
    if (!dq || !dk_out || !dv_out || !dlog_alpha || !dbeta) return -1;
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
        const size_t n = (size_t)dv * dk;
        const long nck = (L + kSeg - 1) / kSeg;
        double *mem = (double *)malloc(sizeof(double) *
                                       (n * (size_t)(nck + kSeg + 2) + 3 * (size_t)dv));
        if (!mem) { bad |= 1; continue; }
        double *ck = mem, *seg = ck + n * (size_t)nck, *G = seg + n * (kSeg + 1);
        double *p = G + n, *du = p + dv, *dp = du + dv;
        const long gk = t0 * H + h;
        const long unit_state = ((long)u * H + h) * (long)n;
        bwd_unit(L, dk, dv, q + gk * dk, k + gk * dk, v + gk * dv, log_alpha + gk, beta + gk,
                 (long)H * dk, (long)H * dv, H,
                 S0 ? S0 + unit_state : NULL, dO + gk * dv, dS_T ? dS_T + unit_state : NULL,
                 dq + gk * dk, dk_out + gk * dk, dv_out + gk * dv, dlog_alpha + gk, dbeta + gk,
                 dS0 ? dS0 + unit_state : NULL, ck, seg, G, p, du, dp);
        free(mem);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * Channel-wise decay (KDA), fp64, token by token.
 *
 * "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
 * (abstract) describes Kimi Delta Attention as the delta rule with
 * channel-wise decay, and states that it reduces to Gated DeltaNet when the
 * decay collapses to a scalar.  The pages print no equation; the reading
 * used here keeps the scalar-gate rule above and lets the gate act on the
 * key channels (the columns of S):
 *
 *     S~  = S_{t-1} Diag(alpha_t)            alpha_t in (0,1]^{d_k}
 *     p   = S~ k_t
 *     S_t = S~ + beta_t (v_t - p) k_t^T,     o_t = S_t q_t
 *
 * which is S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 * and equals the scalar rule when every channel of alpha_t is the same.
 * log_alpha is [B,T,H,d_k]; every other layout is as in gdn_oracle_fwd.
 * ------------------------------------------------------------------------ */
int gdn_oracle_kda_fwd(int B, long T, int H, int dk, int dv,
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
        double *St = (double *)malloc(sizeof(double) * ((size_t)dv * dk + dk));
        if (!St) { bad |= 1; continue; }
        double *decay = St + (size_t)dv * dk;
        const long unit_state = ((long)u * H + h) * dv * dk;
        for (long e = 0; e < (long)dv * dk; ++e) St[e] = S0 ? S0[unit_state + e] : 0.0;
        for (long t = 0; t < L; ++t) {
            const long row = (t0 + t) * H + h;           /* token-head index */
            const double *kt = k + row * dk, *qt = q + row * dk, *vt = v + row * dv;
            const double *lat = log_alpha + row * dk;
            const double b = beta[row];
            for (int c = 0; c < dk; ++c) decay[c] = exp(lat[c]);
            for (int r = 0; r < dv; ++r) {
                double *Sr = St + (long)r * dk;
                double read = 0.0;
                for (int c = 0; c < dk; ++c) {
                    Sr[c] *= decay[c];                   /* S~ = S Diag(alpha) */
                    read += Sr[c] * kt[c];
                }
                const double wr = b * (vt[r] - read);
                double out = 0.0;
                for (int c = 0; c < dk; ++c) {
                    Sr[c] += wr * kt[c];
                    out += Sr[c] * qt[c];
                }
                if (o) o[row * dv + r] = out;
            }
        }
        if (S_T)
            for (long e = 0; e < (long)dv * dk; ++e) S_T[unit_state + e] = St[e];
        free(St);
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * Gated DeltaNet-2, fp64, token by token.
 *
 * "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
 * (abstract): the delta rule's single scalar gate, which sets both how much
 * old content is erased on the key side and how much new content is
 * committed on the value side, is split into a channel-wise erase gate b_t
 * and a channel-wise write gate w_t; with both equal to one scalar the rule
 * is KDA, with a scalar decay too it is Gated DeltaNet.  The pages print no
 * equation; the reading here replaces beta in the erase term of the KDA
 * step by b_t on the key side and beta in the write term by w_t on the
 * value side:
 *
 *     S~  = S_{t-1} Diag(alpha_t)
 *     S_t = S~ - (S~ k_t)(b_t o k_t)^T + (w_t o v_t) k_t^T,   o_t = S_t q_t
 *
 * erase [B,T,H,d_k] holds b_t, write [B,T,H,d_v] holds w_t; log_alpha is
 * [B,T,H,d_k]; every other layout is as in gdn_oracle_fwd.
 * ------------------------------------------------------------------------ */
int gdn_oracle_gdn2_fwd(int B, long T, int H, int dk, int dv,
                        int n_seqs, const int32_t *cu_seqlens,
                        const double *q, const double *k, const double *v,
                        const double *log_alpha, const double *erase, const double *write,
                        const double *S0, double *o, double *S_T, int n_threads)
{
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !log_alpha || !erase || !write) return -1;
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
        double *St = (double *)malloc(sizeof(double) * ((size_t)dv * dk + 2 * (size_t)dk));
        if (!St) { bad |= 1; continue; }
        double *decay = St + (size_t)dv * dk, *ek = decay + dk;
        const long unit_state = ((long)u * H + h) * dv * dk;
        for (long e = 0; e < (long)dv * dk; ++e) St[e] = S0 ? S0[unit_state + e] : 0.0;
        for (long t = 0; t < L; ++t) {
            const long row = (t0 + t) * H + h;
            const double *kt = k + row * dk, *qt = q + row * dk, *vt = v + row * dv;
            const double *lat = log_alpha + row * dk, *bt = erase + row * dk;
            const double *wt = write + row * dv;
            for (int c = 0; c < dk; ++c) {
                decay[c] = exp(lat[c]);
                ek[c] = bt[c] * kt[c];                   /* erase direction b o k */
            }
            for (int r = 0; r < dv; ++r) {
                double *Sr = St + (long)r * dk;
                double rd = 0.0;
                for (int c = 0; c < dk; ++c) {
                    Sr[c] *= decay[c];
                    rd += Sr[c] * kt[c];                 /* read (S~ k)_r */
                }
                const double wv = wt[r] * vt[r];
                double out = 0.0;
                for (int c = 0; c < dk; ++c) {
                    Sr[c] += wv * kt[c] - rd * ek[c];
                    out += Sr[c] * qt[c];
                }
                if (o) o[row * dv + r] = out;
            }
        }
        if (S_T)
            for (long e = 0; e < (long)dv * dk; ++e) S_T[unit_state + e] = St[e];
        free(St);
    }
    return bad ? -1 : 0;
}
