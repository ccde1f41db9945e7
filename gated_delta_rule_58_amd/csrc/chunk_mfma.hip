// Chunkwise forward of the gated delta rule on gfx950 matrix cores (bf16
// inputs, fp32 state and accumulation).
//
// Method: the extended WY/UT chunk algorithm ("Gated Delta Networks:
// Improving Mamba2 with Delta Rule", research-map summary, section
// "Approach"; blog "Gated DeltaNet: Harmonizing Gating and the Delta Rule for
// Superior Linear RNNs", section "Hardware-Efficient Training").  For one
// chunk of C = 64 tokens (zero-padded at a ragged end) and the state S that
// enters it, with g the chunk-local prefix sum of log alpha:
//   (1) g_r = sum_{s<=r} log alpha_s
//   (2) A[r,i] = beta_r e^{g_r-g_i} (k_r . k_i) for i < r;  T = (I + A)^{-1}
//   (3) U = T diag(beta) V,  W = T diag(beta e^g) K
//   (4) Delta = U - W S^T;   S <- e^{g_C} S + Delta^T diag(e^{g_C-g}) K
//   (5) O = diag(e^g) Q S^T + (tril(Q K^T) o e^{g_r-g_i}) Delta
//
// One workgroup (4 waves) owns one (sequence, head, 64-wide slice of d_v)
// and walks the chunks in order, so the whole pass is a single read of
// q, k, v and the gates, and a single write of o; nothing is staged in HBM.
// Per chunk:
//   - stage (1)-(3) are computed cooperatively into LDS: Q K^T and K K^T on
//     MFMA, the 64x64 unit-lower inverse as four 16x16 diagonal blocks by
//     forward substitution in fp32 followed by three bands of 16x16 MFMA
//     block products (T_ij = -T_ii sum_k A_ik T_kj), then W on MFMA;
//   - stage (4)-(5) is wave-local: wave w owns 16 columns of the d_v slice,
//     keeps its S^T columns (d_k x 16, fp32) in MFMA accumulators, and feeds
//     S^T and Delta from accumulator registers straight into the next MFMAs
//     (see gdn_common.h for the register layouts).
// Precision: the outputs are heavy-tailed (max |o| is 10-20x its RMS), so
// plain bf16 operands lose too much.  The operands that carry the state or
// the corrected values are split into hi + lo bf16 pairs (S^T, Delta, P),
// the beta-diagonal of U is applied in fp32, and o is written in fp32 (or
// bf16 on request).
#include "gdn_common.h"

namespace gdn {

constexpr int kC = 64;     // chunk length
constexpr int kDVT = 64;   // d_v columns per workgroup (16 per wave)

template <int DK, typename TO>
__global__ __launch_bounds__(256, 1) void chunk_mfma_kernel(
    int T, int H, int DV, int varlen, int xcd_map, const int32_t *__restrict__ cu_seqlens,
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ S0, TO *__restrict__ o, float *__restrict__ S_T) {
    constexpr int C = kC;
    constexpr int NKS = DK / 32;      // 32-wide k-steps over d_k
    constexpr int NMT = DK / 16;      // 16-row tiles over d_k
    constexpr int NMW = NMT / 4;      // d_k tiles of W^T per wave
    constexpr int LDK = DK + 8;       // padded row lengths (elements)
    constexpr int LDC = C + 8;
    constexpr int LDV = kDVT + 8;
    constexpr int LDA = C + 4;

    __shared__ __attribute__((aligned(16))) bf16 sQ[C * LDK];
    __shared__ __attribute__((aligned(16))) bf16 sK[C * LDK];
    __shared__ __attribute__((aligned(16))) bf16 sV[C * LDV];
    __shared__ __attribute__((aligned(16))) float sA[C * LDA];      // A (strict lower)
    __shared__ __attribute__((aligned(16))) float sAd[4 * 16 * 16]; // diag blocks of A, transposed
    __shared__ __attribute__((aligned(16))) float sT[C * LDA];      // T, later W (bf16)
    __shared__ __attribute__((aligned(16))) bf16 sTU[C * LDC];      // strict-lower T diag(beta)
    __shared__ __attribute__((aligned(16))) bf16 sTW[C * LDC];      // T diag(beta e^g)
    __shared__ __attribute__((aligned(16))) bf16 sPh[C * LDC];      // P = tril(QK^T) o decay, hi
    __shared__ __attribute__((aligned(16))) bf16 sPl[C * LDC];      // P, lo
    __shared__ float sg[C], seg[C], sb[C];
    bf16 *sW = reinterpret_cast<bf16 *>(sT);
    static_assert(C * LDK * sizeof(bf16) <= C * LDA * sizeof(float), "sW must fit in sT");

    // Workgroup -> (unit, head, d_v slice).  With xcd_map the two slices of
    // one (unit, head) land on the same XCD (workgroups are dealt to the 8
    // XCDs round-robin), so the second read of q and k hits that XCD's L2.
    const int ndvt = DV / kDVT;
    int uh, dvt;
    if (xcd_map) {
        const int b = blockIdx.x;
        uh = (b & 7) + 8 * (b / (8 * ndvt));
        dvt = (b >> 3) % ndvt;
    } else {
        uh = blockIdx.x / ndvt;
        dvt = blockIdx.x % ndvt;
    }
    const int unit = uh / H, h = uh % H;
    const int dv0 = dvt * kDVT;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lm = lane & 15, lg = lane >> 4;
    const int cw = 16 * w;              // wave's first column within the slice
    const int dvw = dv0 + cw + lm;      // this lane's d_v column

    long row0, L;
    if (varlen) {
        row0 = cu_seqlens[unit];
        L = (long)cu_seqlens[unit + 1] - row0;
    } else {
        row0 = (long)unit * T;
        L = T;
    }
    const size_t sbase = ((size_t)unit * H + h) * DV * DK;

    // st[mt][j] = S^T[16 mt + 4 lg + j][dvw] = S[dvw][16 mt + 4 lg + j]
    f32x4 st[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        if (S0) {
            const float4 x = *reinterpret_cast<const float4 *>(S0 + sbase + (size_t)dvw * DK +
                                                               16 * mt + 4 * lg);
            st[mt] = f32x4{x.x, x.y, x.z, x.w};
        } else {
            st[mt] = zero4();
        }
    }

    for (long c0 = 0; c0 < L; c0 += C) {
        const int n = (int)((L - c0) < C ? (L - c0) : C);
        __syncthreads();   // the previous chunk is done with every LDS buffer

        // ---- load: q, k rows and the v slice (zero rows past the end) ----
        for (int e = tid; e < C * DK / 8; e += 256) {
            const int r = e / (DK / 8), p = e % (DK / 8);
            bf16x8 qv = {}, kv = {};
            if (r < n) {
                const size_t gi = ((size_t)(row0 + c0 + r) * H + h) * DK + 8 * p;
                qv = *reinterpret_cast<const bf16x8 *>(q + gi);
                kv = *reinterpret_cast<const bf16x8 *>(k + gi);
            }
            *reinterpret_cast<bf16x8 *>(sQ + r * LDK + 8 * p) = qv;
            *reinterpret_cast<bf16x8 *>(sK + r * LDK + 8 * p) = kv;
        }
        for (int e = tid; e < C * kDVT / 8; e += 256) {
            const int r = e / (kDVT / 8), p = e % (kDVT / 8);
            bf16x8 vv = {};
            if (r < n)
                vv = *reinterpret_cast<const bf16x8 *>(
                    v + ((size_t)(row0 + c0 + r) * H + h) * DV + dv0 + 8 * p);
            *reinterpret_cast<bf16x8 *>(sV + r * LDV + 8 * p) = vv;
        }
        // ---- (1) gate prefix: one wave, one token per lane ----
        if (w == 0) {
            float x = 0.f, bb = 0.f;
            if (lane < n) {
                const size_t gi = (size_t)(row0 + c0 + lane) * H + h;
                x = log_alpha[gi];
                bb = beta[gi];
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            sg[lane] = x;
            seg[lane] = expf(x);
            sb[lane] = bb;
        }
        __syncthreads();

        // ---- (2a) K K^T and Q K^T, tile row w (r in [16w, 16w+16)) ----
        {
            bf16x8 fKw[NKS], fQw[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                fKw[ks] = frag_rows(sK, LDK, 16 * w, 32 * ks, lane);
                fQw[ks] = frag_rows(sQ, LDK, 16 * w, 32 * ks, lane);
            }
            const int r = 16 * w + lm;
            const float gr = sg[r], br = sb[r];
            for (int tj = 0; tj < 4; ++tj) {
                const int i0 = 16 * tj + 4 * lg;
                if (tj > w) {   // above the diagonal: P is zero there
                    *reinterpret_cast<bf16x4 *>(sPh + r * LDC + i0) = bf16x4{};
                    *reinterpret_cast<bf16x4 *>(sPl + r * LDC + i0) = bf16x4{};
                    continue;
                }
                f32x4 G = zero4(), PT = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 fKj = frag_rows(sK, LDK, 16 * tj, 32 * ks, lane);
                    G = mfma32(fKj, fKw[ks], G);     // (k_i . k_r), i = i0 + j
                    PT = mfma32(fKj, fQw[ks], PT);   // (k_i . q_r)
                }
                f32x4 a4;
                bf16x4 ph, pl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j;
                    const float dec = (i <= r) ? expf(gr - sg[i]) : 0.f;
                    a4[j] = (i < r) ? br * dec * G[j] : 0.f;
                    const float p = dec * PT[j];
                    ph[j] = (bf16)p;
                    pl[j] = (bf16)(p - (float)ph[j]);
                }
                *reinterpret_cast<f32x4 *>(sA + r * LDA + i0) = a4;
                *reinterpret_cast<bf16x4 *>(sPh + r * LDC + i0) = ph;
                *reinterpret_cast<bf16x4 *>(sPl + r * LDC + i0) = pl;
                if (tj == w) {
                    // K K^T is symmetric: the same registers hold the diagonal
                    // block with rows rr = i0 + j, column ii = r; store it
                    // transposed (column ii contiguous) for the substitution.
                    f32x4 d4;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int rr = i0 + j;
                        d4[j] = (rr > r) ? sb[rr] * expf(sg[rr] - gr) * G[j] : 0.f;
                    }
                    *reinterpret_cast<f32x4 *>(sAd + (16 * w + lm) * 16 + 4 * lg) = d4;
                }
            }
        }
        __syncthreads();

        // ---- (2b) diagonal 16x16 blocks of T by forward substitution (fp32) ----
        {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == lm) ? 1.f : 0.f;
            const float *Ad = sAd + w * 256;
#pragma unroll
            for (int i = 0; i < 15; ++i) {
                float col[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const float4 c4 = *reinterpret_cast<const float4 *>(Ad + i * 16 + 4 * q4);
                    col[4 * q4] = c4.x;
                    col[4 * q4 + 1] = c4.y;
                    col[4 * q4 + 2] = c4.z;
                    col[4 * q4 + 3] = c4.w;
                }
#pragma unroll
                for (int r = i + 1; r < 16; ++r) x[r] -= col[r] * x[i];
            }
            if (lg == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sT[(16 * w + r) * LDA + 16 * w + lm] = x[r];
            }
        }
        __syncthreads();

        // ---- (2c) off-diagonal blocks, band by band: T_wj = -T_ww sum_k A_wk T_kj ----
        for (int d = 1; d < 4; ++d) {
            if (w >= d) {
                const int jb = w - d;
                f32x4 Y = zero4();
                for (int kk = jb; kk < w; ++kk) {
                    const float4 av = *reinterpret_cast<const float4 *>(
                        sA + (16 * w + lm) * LDA + 16 * kk + 4 * lg);
                    const bf16x4 aop = {(bf16)av.x, (bf16)av.y, (bf16)av.z, (bf16)av.w};
                    bf16x4 bop;
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        bop[s] = (bf16)sT[(16 * kk + 4 * lg + s) * LDA + 16 * jb + lm];
                    Y = mfma16(aop, bop, Y);
                }
                const float4 tv = *reinterpret_cast<const float4 *>(
                    sT + (16 * w + lm) * LDA + 16 * w + 4 * lg);
                const bf16x4 top = {(bf16)tv.x, (bf16)tv.y, (bf16)tv.z, (bf16)tv.w};
                const bf16x4 yop = {(bf16)Y[0], (bf16)Y[1], (bf16)Y[2], (bf16)Y[3]};
                const f32x4 R = mfma16(top, yop, zero4());
#pragma unroll
                for (int j = 0; j < 4; ++j) sT[(16 * w + 4 * lg + j) * LDA + 16 * jb + lm] = -R[j];
            }
            __syncthreads();
        }

        // ---- (3a) T diag(beta) (strictly lower) and T diag(beta e^g) in bf16 ----
        for (int e = tid; e < C * C / 4; e += 256) {
            const int r = e / (C / 4), c4 = 4 * (e % (C / 4));
            const float4 tv = *reinterpret_cast<const float4 *>(sT + r * LDA + c4);
            const float t[4] = {tv.x, tv.y, tv.z, tv.w};
            bf16x4 tu, tw;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int c = c4 + s;
                tu[s] = (bf16)((c < r) ? t[s] * sb[c] : 0.f);
                tw[s] = (bf16)((c <= r) ? t[s] * sb[c] * seg[c] : 0.f);
            }
            *reinterpret_cast<bf16x4 *>(sTU + r * LDC + c4) = tu;
            *reinterpret_cast<bf16x4 *>(sTW + r * LDC + c4) = tw;
        }
        __syncthreads();

        // ---- (3b) W^T = K^T (T diag(beta e^g))^T, d_k rows [16 NMW w, +16 NMW) ----
#pragma unroll
        for (int mi = 0; mi < NMW; ++mi) {
            const int mt = w * NMW + mi;
            const bf16x8 fKT0 = frag_cols(sK, LDK, 16 * mt, 0, lane);
            const bf16x8 fKT1 = frag_cols(sK, LDK, 16 * mt, 32, lane);
#pragma unroll
            for (int nr = 0; nr < 4; ++nr) {
                f32x4 acc = mfma32(fKT0, frag_rows(sTW, LDC, 16 * nr, 0, lane), zero4());
                if (nr >= 2) acc = mfma32(fKT1, frag_rows(sTW, LDC, 16 * nr, 32, lane), acc);
                // acc[j] = W[16 nr + lm][16 mt + 4 lg + j]
                const bf16x4 wv = {(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
                *reinterpret_cast<bf16x4 *>(sW + (16 * nr + lm) * LDK + 16 * mt + 4 * lg) = wv;
            }
        }
        // ---- (3c) U for the wave's 16 columns: beta V (fp32) + strict-lower part ----
        f32x4 U[4];
        {
            const bf16x8 fV0 = frag_cols(sV, LDV, cw, 0, lane);
            const bf16x8 fV1 = frag_cols(sV, LDV, cw, 32, lane);
#pragma unroll
            for (int mr = 0; mr < 4; ++mr) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * mr + 4 * lg + j;
                    U[mr][j] = sb[r] * (float)sV[r * LDV + cw + lm];
                }
                U[mr] = mfma32(frag_rows(sTU, LDC, 16 * mr, 0, lane), fV0, U[mr]);
                if (mr >= 2) U[mr] = mfma32(frag_rows(sTU, LDC, 16 * mr, 32, lane), fV1, U[mr]);
            }
        }
        __syncthreads();   // W complete

        // ---- (4)-(5) wave-local: Delta, O, state update ----
        bf16x8 sh[NKS], sl[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) split_op(st[2 * ks], st[2 * ks + 1], sh[ks], sl[ks]);

        f32x4 D[4], O[4];
#pragma unroll
        for (int mr = 0; mr < 4; ++mr) {
            f32x4 ws = zero4(), qs = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 fw = frag_rows_d(sW, LDK, 16 * mr, 32 * ks, lane);
                ws = mfma32(fw, sh[ks], ws);
                ws = mfma32(fw, sl[ks], ws);
                const bf16x8 fq = frag_rows_d(sQ, LDK, 16 * mr, 32 * ks, lane);
                qs = mfma32(fq, sh[ks], qs);
                qs = mfma32(fq, sl[ks], qs);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                D[mr][j] = U[mr][j] - ws[j];
                O[mr][j] = seg[16 * mr + 4 * lg + j] * qs[j];
            }
        }
        bf16x8 dh[2], dl[2];
        split_op(D[0], D[1], dh[0], dl[0]);
        split_op(D[2], D[3], dh[1], dl[1]);
#pragma unroll
        for (int mr = 0; mr < 4; ++mr) {
#pragma unroll
            for (int ks = 0; ks <= mr / 2; ++ks) {
                const bf16x8 fph = frag_rows_d(sPh, LDC, 16 * mr, 32 * ks, lane);
                const bf16x8 fpl = frag_rows_d(sPl, LDC, 16 * mr, 32 * ks, lane);
                O[mr] = mfma32(fph, dh[ks], O[mr]);
                O[mr] = mfma32(fpl, dh[ks], O[mr]);
                O[mr] = mfma32(fph, dl[ks], O[mr]);
            }
        }
#pragma unroll
        for (int mr = 0; mr < 4; ++mr) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * mr + 4 * lg + j;
                if (r < n) o[((size_t)(row0 + c0 + r) * H + h) * DV + dvw] = from_f32<TO>(O[mr][j]);
            }
        }

        const float gC = sg[C - 1];
        bf16x8 th[2], tl[2];
        {
            f32x4 Dt[4];
#pragma unroll
            for (int mr = 0; mr < 4; ++mr)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    Dt[mr][j] = D[mr][j] * expf(gC - sg[16 * mr + 4 * lg + j]);
            split_op(Dt[0], Dt[1], th[0], tl[0]);
            split_op(Dt[2], Dt[3], th[1], tl[1]);
        }
        const float egC = seg[C - 1];
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
            st[mt] = st[mt] * egC;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 fk = frag_cols_d(sK, LDK, 16 * mt, 32 * ks, lane);
                st[mt] = mfma32(fk, th[ks], st[mt]);
                st[mt] = mfma32(fk, tl[ks], st[mt]);
            }
        }
    }

    if (S_T) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
            *reinterpret_cast<float4 *>(S_T + sbase + (size_t)dvw * DK + 16 * mt + 4 * lg) =
                float4{st[mt][0], st[mt][1], st[mt][2], st[mt][3]};
    }
}

bool chunk_mfma_supported(int dk, int dv, int chunk) {
    return chunk == kC && dk == dv && (dk == 64 || dk == 128);
}

template <int DK, typename TO>
hipError_t launch_chunk_mfma_t(int units, int T, int H, int DV, const int32_t *cu,
                               const void *q, const void *k, const void *v,
                               const float *la, const float *beta, const float *S0,
                               void *o, float *S_T, hipStream_t st) {
    const int ndvt = DV / kDVT;
    const long nwg = (long)units * H * ndvt;
    const int xcd_map = ((long)units * H) % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((chunk_mfma_kernel<DK, TO>), dim3((unsigned)nwg), dim3(256), 0, st,
                       T, H, DV, cu != nullptr ? 1 : 0, xcd_map, cu, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)v, la, beta, S0, (TO *)o, S_T);
    return hipGetLastError();
}

hipError_t launch_chunk_mfma(int units, int T, int H, int dk, bool o_bf16, const int32_t *cu,
                             const void *q, const void *k, const void *v, const float *la,
                             const float *beta, const float *S0, void *o, float *S_T,
                             hipStream_t st) {
    if (dk == 128)
        return o_bf16 ? launch_chunk_mfma_t<128, bf16>(units, T, H, dk, cu, q, k, v, la, beta, S0, o, S_T, st)
                      : launch_chunk_mfma_t<128, float>(units, T, H, dk, cu, q, k, v, la, beta, S0, o, S_T, st);
    if (dk == 64)
        return o_bf16 ? launch_chunk_mfma_t<64, bf16>(units, T, H, dk, cu, q, k, v, la, beta, S0, o, S_T, st)
                      : launch_chunk_mfma_t<64, float>(units, T, H, dk, cu, q, k, v, la, beta, S0, o, S_T, st);
    return hipErrorInvalidValue;
}

}  // namespace gdn
