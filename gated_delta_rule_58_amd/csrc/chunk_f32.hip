// Chunkwise forward of the gated delta rule in fp32 on the vector ALUs.
//
// This is the fp32-I/O instance of the extended WY/UT chunk algorithm
// ("Gated Delta Networks: Improving Mamba2 with Delta Rule", research-map
// summary, section "Approach"; blog "Gated DeltaNet: Harmonizing Gating and
// the Delta Rule for Superior Linear RNNs", section "Hardware-Efficient
// Training").  It exists for inputs that must stay fp32 end to end (small
// head widths, tight tolerances); the bf16 MFMA kernel handles the large
// shapes.  For one chunk of n <= C tokens and the state S (d_v x d_k) that
// enters it, with g the chunk-local prefix sum of log alpha:
//   A[r,i] = beta_r e^{g_r - g_i} (k_r . k_i)  (i < r),  T = (I + A)^{-1}
//   U = T diag(beta) V,  W = T diag(beta e^g) K,  Delta = U - W S^T
//   O = diag(e^g) Q S^T + (tril(Q K^T) o e^{g_r - g_i}) Delta
//   S <- e^{g_n} S + Delta^T diag(e^{g_n - g}) K
// Only exponentials of non-positive arguments are formed.
//
// One 256-thread workgroup per (sequence, head) walks its chunks in order;
// every intermediate lives in LDS.  With the input prologue, q and k rows are
// L2-normalised in LDS after loading (norm clamped below at 1e-6) and the
// gates arrive as pre-activations a, b: log alpha = -softplus(a),
// beta = sigmoid(b).
#include "gdn_common.h"

namespace gdn {

template <int DK, int DV, int C, typename TO>
__global__ __launch_bounds__(256) void chunk_f32_kernel(
    int T, int H, int varlen, int norm_qk, int gates, const int32_t *__restrict__ cu_seqlens,
    const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ log_alpha,
    const float *__restrict__ beta, const float *__restrict__ S0,
    TO *__restrict__ o, float *__restrict__ S_T) {
    __shared__ float sK[C][DK], sQ[C][DK], sW[C][DK];
    __shared__ float sV[C][DV], sU[C][DV];
    __shared__ float sS[DV][DK];
    __shared__ float sA[C][C + 1], sT[C][C + 1], sP[C][C + 1];
    __shared__ float sg[C], sb[C];

    const int unit = blockIdx.x / H, h = blockIdx.x % H;
    const int tid = threadIdx.x;
    long row0, L;
    if (varlen) {
        row0 = cu_seqlens[unit];
        L = (long)cu_seqlens[unit + 1] - row0;
    } else {
        row0 = (long)unit * T;
        L = T;
    }
    const size_t state_off = ((size_t)unit * H + h) * DV * DK;

    for (int e = tid; e < DV * DK; e += 256)
        sS[e / DK][e % DK] = S0 ? S0[state_off + e] : 0.f;

    for (long c0 = 0; c0 < L; c0 += C) {
        const int n = (int)((L - c0) < C ? (L - c0) : C);
        __syncthreads();   // previous chunk done with LDS
        for (int e = tid; e < n * DK; e += 256) {
            const int r = e / DK, i = e % DK;
            const size_t g = ((size_t)(row0 + c0 + r) * H + h) * DK + i;
            sK[r][i] = k[g];
            sQ[r][i] = q[g];
        }
        for (int e = tid; e < n * DV; e += 256) {
            const int r = e / DV, i = e % DV;
            sV[r][i] = v[((size_t)(row0 + c0 + r) * H + h) * DV + i];
        }
        if (tid < n) {
            const size_t g = (size_t)(row0 + c0 + tid) * H + h;
            float a = log_alpha[g], b = beta[g];
            if (gates) {
                a = -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a))));
                b = 1.f / (1.f + expf(-b));
            }
            sg[tid] = a;
            sb[tid] = b;
        }
        __syncthreads();
        if (norm_qk && tid < 2 * n) {   // one thread per q or k row
            float *x = tid < n ? sQ[tid] : sK[tid - n];
            float ss = 0.f;
            for (int d = 0; d < DK; ++d) ss += x[d] * x[d];
            const float inv = 1.f / sqrtf(fmaxf(ss, 1e-12f));
            for (int d = 0; d < DK; ++d) x[d] *= inv;
        }
        if (tid == 0)   // chunk-local prefix sum of log alpha
            for (int r = 1; r < n; ++r) sg[r] += sg[r - 1];
        __syncthreads();

        // A (strict lower) and P = tril(Q K^T) o decay (diagonal kept)
        for (int e = tid; e < n * n; e += 256) {
            const int r = e / n, i = e % n;
            float a = 0.f, p = 0.f;
            if (i <= r) {
                float kk = 0.f, qk = 0.f;
                for (int d = 0; d < DK; ++d) {
                    kk += sK[r][d] * sK[i][d];
                    qk += sQ[r][d] * sK[i][d];
                }
                const float dec = expf(sg[r] - sg[i]);
                if (i < r) a = sb[r] * dec * kk;
                p = dec * qk;
            }
            sA[r][i] = a;
            sP[r][i] = p;
        }
        __syncthreads();

        // T = (I + A)^{-1}: column j by forward substitution
        if (tid < n) {
            const int j = tid;
            for (int r = 0; r < j; ++r) sT[r][j] = 0.f;
            sT[j][j] = 1.f;
            for (int r = j + 1; r < n; ++r) {
                float acc = 0.f;
                for (int i = j; i < r; ++i) acc += sA[r][i] * sT[i][j];
                sT[r][j] = -acc;
            }
        }
        __syncthreads();

        // U = T diag(beta) V,  W = T diag(beta e^g) K
        for (int e = tid; e < n * DV; e += 256) {
            const int r = e / DV, c = e % DV;
            float acc = 0.f;
            for (int i = 0; i <= r; ++i) acc += sT[r][i] * sb[i] * sV[i][c];
            sU[r][c] = acc;
        }
        for (int e = tid; e < n * DK; e += 256) {
            const int r = e / DK, d = e % DK;
            float acc = 0.f;
            for (int i = 0; i <= r; ++i) acc += sT[r][i] * sb[i] * expf(sg[i]) * sK[i][d];
            sW[r][d] = acc;
        }
        __syncthreads();

        // Delta = U - W S^T (in place over U)
        for (int e = tid; e < n * DV; e += 256) {
            const int r = e / DV, c = e % DV;
            float acc = 0.f;
            for (int d = 0; d < DK; ++d) acc += sW[r][d] * sS[c][d];
            sU[r][c] -= acc;
        }
        __syncthreads();

        // O = diag(e^g) Q S^T + P Delta
        for (int e = tid; e < n * DV; e += 256) {
            const int r = e / DV, c = e % DV;
            float qs = 0.f, pd = 0.f;
            for (int d = 0; d < DK; ++d) qs += sQ[r][d] * sS[c][d];
            for (int i = 0; i <= r; ++i) pd += sP[r][i] * sU[i][c];
            o[((size_t)(row0 + c0 + r) * H + h) * DV + c] =
                from_f32<TO>(expf(sg[r]) * qs + pd);
        }
        __syncthreads();

        // S <- e^{g_n} S + Delta^T diag(e^{g_n - g}) K
        const float gn = sg[n - 1];
        for (int e = tid; e < DV * DK; e += 256) {
            const int c = e / DK, d = e % DK;
            float acc = 0.f;
            for (int r = 0; r < n; ++r) acc += sU[r][c] * expf(gn - sg[r]) * sK[r][d];
            sS[c][d] = expf(gn) * sS[c][d] + acc;
        }
    }
    __syncthreads();
    if (S_T)
        for (int e = tid; e < DV * DK; e += 256) S_T[state_off + e] = sS[e / DK][e % DK];
}

template <int DK, int C, typename TO>
hipError_t launch_chunk_f32_t(int units, int T, int H, int norm_qk, int gates, const int32_t *cu,
                              const void *q, const void *k, const void *v,
                              const float *la, const float *beta, const float *S0,
                              void *o, float *S_T, hipStream_t st) {
    hipLaunchKernelGGL((chunk_f32_kernel<DK, DK, C, TO>), dim3(units * H), dim3(256),
                       0, st, T, H, cu != nullptr ? 1 : 0, norm_qk, gates, cu, (const float *)q,
                       (const float *)k, (const float *)v, la, beta, S0, (TO *)o, S_T);
    return hipGetLastError();
}

// d_k = d_v = dk in {16, 32, 64}, chunk in {16, 32, 64}; fp32 q,k,v.
bool chunk_f32_supported(int dk, int dv, int chunk) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64) &&
           (chunk == 16 || chunk == 32 || chunk == 64);
}

hipError_t launch_chunk_f32(int units, int T, int H, int dk, int chunk, bool o_bf16,
                            bool norm_qk, bool gates,
                            const int32_t *cu, const void *q, const void *k,
                            const void *v, const float *la, const float *beta,
                            const float *S0, void *o, float *S_T, hipStream_t st) {
#define GDN_F32_CASE(DKV, CV)                                                        \
    if (dk == DKV && chunk == CV)                                                    \
        return o_bf16 ? launch_chunk_f32_t<DKV, CV, bf16>(units, T, H, norm_qk, gates, cu, \
                                                          q, k, v, la, beta, S0, o, S_T, st) \
                      : launch_chunk_f32_t<DKV, CV, float>(units, T, H, norm_qk, gates, cu, \
                                                           q, k, v, la, beta, S0, o, S_T, st);
    GDN_F32_CASE(16, 16) GDN_F32_CASE(16, 32) GDN_F32_CASE(16, 64)
    GDN_F32_CASE(32, 16) GDN_F32_CASE(32, 32) GDN_F32_CASE(32, 64)
    GDN_F32_CASE(64, 16) GDN_F32_CASE(64, 32) GDN_F32_CASE(64, 64)
#undef GDN_F32_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
