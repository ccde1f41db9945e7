// Gated DeltaNet-2 forward on gfx950 (fp32 MFMA): channel-wise decay with a
// channel-wise erase gate on the key side and a write gate on the value side.
//
// "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
// (abstract) splits the delta rule's single scalar gate into an erase gate
// b_t and a write gate w_t, reducing to KDA when both are one scalar; the
// pages print no equation.  The rule computed here:
//
//   S~  = S_{t-1} Diag(alpha_t),   S_t = S~ - (S~ k_t)(b_t o k_t)^T + (w_t o v_t) k_t^T,
//   o_t = S_t q_t.
//
// Chunk form (G the per-channel prefix of log alpha, E = B o K, Z = W o V,
// every channel weight e^{G_rc - G_ic} with i <= r):
//   A_e[r,i] = sum_c k_rc e_ic e^{..},  A_k[r,i] = sum_c k_rc k_ic e^{..}   (i < r)
//   P_e, P_k: the same with q_r, i <= r;   T_e = (I + A_e)^{-1}
//   X  = -T_e ((K o e^G) S^T + A_k Z)          (the erased reads, rows x_r)
//   O  = (Q o e^G) S^T + P_e X + P_k Z
//   S' = S Diag(e^{G_n}) + X^T (E o e^{G_n - G}) + Z^T (K o e^{G_n - G})
// Folding the state-independent factors in a prep launch,
//   F1 = T_e (K o e^G),  N1 = T_e A_k,  M = P_e T_e,
//   Qh = Q o e^G - M (K o e^G),  N2 = P_k - M A_k,
// leaves the sequential launch X = -(F1 S^T + N1 Z), O = Qh S^T + N2 Z and the
// state update.
#include "fp32_tiles.h"

namespace gdn {
namespace {

using namespace tiles;


// Workspace blocks (floats) per chunk and head.
template <int D> struct G2Ws {
    static constexpr size_t N1 = BC * BC, N2 = BC * BC, F1 = BC * D, QH = BC * D, ET = BC * D,
                            KT = BC * D, EG = D;
    static constexpr size_t total = N1 + N2 + F1 + QH + ET + KT + EG;
    static constexpr size_t oN1 = 0, oN2 = N1, oF1 = oN2 + N2, oQH = oF1 + F1, oET = oQH + QH,
                            oKT = oET + ET, oEG = oKT + KT;
};

// ---------------------------------------------------------------- 1. prep
template <int D, typename TI>
__global__ __launch_bounds__(512) void gdn2_prep_kernel(
    int T, int H, int units, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ q, const TI *__restrict__ k, const float *__restrict__ la,
    const float *__restrict__ erase, float *__restrict__ ws, int nch) {
    constexpr int LI = ldx<TI, D>(), LF = D + 4, LE = D + 8;
    constexpr int NE = BC * LE > 2 * BC * LDN ? BC * LE : 2 * BC * LDN;   // E, then A_e | A_k
    __shared__ __attribute__((aligned(16))) TI sK[BC * LI];
    __shared__ __attribute__((aligned(16))) TI sQ[BC * LI];
    __shared__ __attribute__((aligned(16))) float sG[BC * LF];   // per-channel prefix G
    __shared__ __attribute__((aligned(16))) float sE[NE];   // b o k, then A_e (-> M) | A_k
    __shared__ __attribute__((aligned(16))) float sPe[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sPk[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sTe[BC * LDN];
    float *sAe = sE, *sAk = sE + BC * LDN;
    const int tid = threadIdx.x, wave = tid >> 6;
    // Persistent over the (chunk slot, head) pairs ci = blockIdx.x + j gridDim.x:
    // the inputs of the next pair load into registers while this one is
    // computed.
    Prefetch<D, TI> pk, pq;
    Prefetch<D, float> pg, pe;
    auto next = [&](int c) {   // first pair >= c with a chunk (unused slots skipped), and fetch it
        long r0;
        int nv;
        for (; c < nch; c += gridDim.x) {
            if (!slot_chunk(c / H, units, T, NC, varlen, cu, r0, nv)) continue;
            const size_t g0 = (size_t)r0 * H * D + (size_t)(c % H) * D;
            pk.fetch(k + g0, (size_t)H * D, nv, tid);
            pq.fetch(q + g0, (size_t)H * D, nv, tid);
            pg.fetch(la + g0, (size_t)H * D, nv, tid);
            pe.fetch(erase + g0, (size_t)H * D, nv, tid);
            break;
        }
        return c;
    };
    for (int ci = next(blockIdx.x); ci < nch;) {
    // the lane index passes through an empty asm statement each iteration, so
    // the per-lane LDS addresses below are recomputed rather than hoisted out
    // of the loop and kept live in registers across it
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    const int li = lane & 15, lq = lane >> 4;
    float *W = ws + (size_t)ci * G2Ws<D>::total;
    pk.commit(sK, LI, tid);
    pq.commit(sQ, LI, tid);
    pg.commit(sG, LF, tid);
    pe.commit(sE, LE, tid);
    for (int e = tid; e < BC * LDN; e += 512) sTe[e] = 0.f;
    __syncthreads();
    const int cn = next(ci + gridDim.x);
    if (tid < D) {   // prefix over the chunk per channel (padded rows add 0)
        float g = 0.f;
        for (int r = 0; r < BC; ++r) {
            g += sG[r * LF + tid];
            sG[r * LF + tid] = g;
        }
        W[G2Ws<D>::oEG + tid] = expf(g);
    }
    for (int e = tid; e < BC * D / 4; e += 512) {   // E = b o k
        const int r = e / (D / 4), c = (e % (D / 4)) * 4;
        const f32x4 kv = ld4f(sK + r * LI + c);
        f32x4 *pe = reinterpret_cast<f32x4 *>(sE + r * LE + c);
        *pe = *pe * kv;
    }
    __syncthreads();
    // E o e^{G_n - G} and K o e^{G_n - G} for the state update
    for (int e = tid; e < BC * D / 4; e += 512) {
        const int r = e / (D / 4), c = (e % (D / 4)) * 4;
        const f32x4 g = *reinterpret_cast<const f32x4 *>(sG + r * LF + c);
        const f32x4 gn = *reinterpret_cast<const f32x4 *>(sG + (BC - 1) * LF + c);
        const f32x4 kv = ld4f(sK + r * LI + c);
        const f32x4 ev = *reinterpret_cast<const f32x4 *>(sE + r * LE + c);
        f32x4 et, kt;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float t = __expf(gn[j] - g[j]);
            et[j] = ev[j] * t;
            kt[j] = kv[j] * t;
        }
        *reinterpret_cast<f32x4 *>(W + G2Ws<D>::oET + 4 * e) = et;
        *reinterpret_cast<f32x4 *>(W + G2Ws<D>::oKT + 4 * e) = kt;
    }
    // The four channel-weighted products, 16 x 16 blocks (br, bi), bi <= br:
    // matrix mx = 0 A_e (rows K, columns E), 1 A_k (K, K), 2 P_e (Q, E),
    // 3 P_k (Q, K).  40 tasks, 5 per wave (2 diagonal, 3 below): waves 0-3
    // the E-column matrices, waves 4-7 the K-column ones.  Each block is one
    // MFMA product of operands rescaled to the prefix just before block br
    // (the last token of block br - 1, or 0): every factor is e^{<= 0} below
    // the diagonal, and on it too unless the block's decay span exceeds 60,
    // when the block is formed term by term instead.  The wave's five
    // chains run interleaved, one MFMA of each per channel step.
    f32x4 res[5];
    {
        const int half = wave >> 2, w4 = wave & 3;   // half 0: E columns, 1: K columns
        int ra[5], rb[5], gro[5], mxs[5];
        float gon[5];
        bool terms[5];
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            const int e = w4 + 4 * s;   // 0..19 within the half
            int blk = e % 10, br = 0;
            while (blk > br) blk -= ++br;
            mxs[s] = 2 * (e / 10) + half;
            ra[s] = 16 * br + li;
            rb[s] = 16 * blk + li;
            gro[s] = br > 0 ? 16 * br - 1 : 0;
            gon[s] = br > 0 ? 1.f : 0.f;   // reference prefix 0 for the first block
            terms[s] = blk == br && diag_span<D>(sG, LF, br, lane) > 60.f;
        }
        auto chains = [&](const auto *Y, int ly) {
#pragma unroll
            for (int s = 0; s < 5; ++s) res[s] = zero4();
#pragma unroll 2
            for (int c0 = 0; c0 < D; c0 += 4) {
                const int c = c0 + lq;
#pragma unroll
                for (int s = 0; s < 5; ++s) {
                    const float gr = gon[s] * sG[gro[s] * LF + c];
                    const TI *Xr = mxs[s] < 2 ? sK : sQ;
                    const float a = to_f32(Xr[ra[s] * LI + c]) * __expf(sG[ra[s] * LF + c] - gr);
                    const float y = to_f32(Y[rb[s] * ly + c]) * __expf(gr - sG[rb[s] * LF + c]);
                    res[s] = mfma_f32(a, y, res[s]);
                }
            }
#pragma unroll
            for (int s = 0; s < 5; ++s)
                if (terms[s])
                    res[s] = diag_terms<D>(mxs[s] < 2 ? sK : sQ, LI, Y, ly, sG, LF, (ra[s] - li) / 16, lane);
        };
        if (half == 0) chains(static_cast<const float *>(sE), LE);
        else chains(static_cast<const TI *>(sK), LI);
        // keep strict (A) or inclusive (P) lower entries
#pragma unroll
        for (int s = 0; s < 5; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = ra[s] - li + 4 * lq + j, i = rb[s];
                if (mxs[s] < 2 ? i >= r : i > r) res[s][j] = 0.f;
            }
    }
    __syncthreads();   // E consumed: A_e and A_k go over it
    for (int e = tid; e < 2 * BC * LDN; e += 512) sE[e] = 0.f;
    for (int e = tid; e < BC * LDN; e += 512) {
        sPe[e] = 0.f;
        sPk[e] = 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        const int e = (wave & 3) + 4 * s, mx = 2 * (e / 10) + (wave >> 2);
        int blk = e % 10, br = 0;
        while (blk > br) blk -= ++br;
        float *dst = mx == 0 ? sAe : mx == 1 ? sAk : mx == 2 ? sPe : sPk;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(16 * br + 4 * lq + j) * LDN + 16 * blk + li] = res[s][j];
    }
    __syncthreads();
    block_inverse64(sAe, sTe, wave, lane);   // T_e (ends with a barrier)
    // M = P_e T_e (over A_e) and N1 = T_e A_k (to the workspace)
    const int ty = wave & 3, tx0 = 2 * (wave >> 2);
    {
        f32x4 m[2], n1[2];
        zero_n(m);
        zero_n(n1);
        mmn<BC, 2>(sPe + 16 * ty * LDN, LDN, 1, sTe + 16 * tx0, LDN, 1, 16, m, lane);
        mmn<BC, 2>(sTe + 16 * ty * LDN, LDN, 1, sAk + 16 * tx0, LDN, 1, 16, n1, lane);
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * ty + 4 * lq + j, c = 16 * (tx0 + x) + li;
                sAe[r * LDN + c] = m[x][j];
                W[G2Ws<D>::oN1 + r * BC + c] = n1[x][j];
            }
    }
    __syncthreads();
    float *sM = sAe;
    {   // N2 = P_k - M A_k
        f32x4 n2[2];
        zero_n(n2);
        mmn<BC, 2>(sM + 16 * ty * LDN, LDN, 1, sAk + 16 * tx0, LDN, 1, 16, n2, lane);
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * ty + 4 * lq + j, c = 16 * (tx0 + x) + li;
                W[G2Ws<D>::oN2 + r * BC + c] = sPk[r * LDN + c] - n2[x][j];
            }
    }
    // F1 = T_e (K o e^G) and Qh = Q o e^G - M (K o e^G), with K o e^G formed
    // in the operand reads; 64 x D tiles, row tr, columns tc0..
    {
        constexpr int NTC = D / 32;
        const int tr = wave & 3, tc0 = (wave >> 2) * NTC;
        f32x4 f1[NTC], qh[NTC];
        zero_n(f1);
        zero_n(qh);
#pragma unroll 4
        for (int kk = 0; kk < BC; kk += 4) {
            const int kr = kk + lq;
            const float a1 = sTe[(16 * tr + li) * LDN + kr];
            const float a2 = sM[(16 * tr + li) * LDN + kr];
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const int c = 16 * (tc0 + t) + li;
                const float b = to_f32(sK[kr * LI + c]) * __expf(sG[kr * LF + c]);
                f1[t] = mfma_f32(a1, b, f1[t]);
                qh[t] = mfma_f32(a2, b, qh[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < NTC; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * tr + 4 * lq + j, c = 16 * (tc0 + t) + li;
                W[G2Ws<D>::oF1 + r * D + c] = f1[t][j];
                W[G2Ws<D>::oQH + r * D + c] =
                    to_f32(sQ[r * LI + c]) * __expf(sG[r * LF + c]) - qh[t][j];
            }
    }
    __syncthreads();   // every LDS operand consumed before the next pair's commit
    ci = cn;
    }
}

// ---------------------------------------------------------------- 2. fwd
template <int D, typename TI, typename TO>
__global__ __launch_bounds__(512) void gdn2_fwd_kernel(
    int T, int H, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ v, const float *__restrict__ write, const float *__restrict__ S0,
    const float *__restrict__ ws, TO *__restrict__ o, float *__restrict__ S_T) {
    constexpr int LF = D + 4, NTC = D / 32, NSL = D / 64;
    __shared__ __attribute__((aligned(16))) float sX1[BC * LF];   // F1, then E o e^{G_n - G}
    __shared__ __attribute__((aligned(16))) float sX2[BC * LF];   // Qh, then K o e^{G_n - G}
    __shared__ __attribute__((aligned(16))) float sS[BC * LF];    // state slice: d_v rows x d_k
    __shared__ __attribute__((aligned(16))) float sZ[BC * LDN];   // Z = w o v (slice)
    __shared__ __attribute__((aligned(16))) float sX[BC * LDN];   // X (erased reads, slice)
    __shared__ float seg[D];
    const int uh = blockIdx.x / NSL, dv0 = 64 * (blockIdx.x % NSL);
    const int u = uh / H, h = uh % H;
    long start, L;
    unit_span(u, T, varlen, cu, start, L);
    const int N = (int)((L + BC - 1) / BC);
    const int base = unit_base(u, NC, varlen, cu);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int tr = wave & 3, tc0 = (wave >> 2) * NTC;
    const int ty = wave & 3, tx0 = 2 * (wave >> 2);
    f32x4 st[NTC];
#pragma unroll
    for (int t = 0; t < NTC; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
            st[t][j] = S0 ? S0[((size_t)uh * D + dv0 + row) * D + col] : 0.f;
        }
    Prefetch<D, float> pf1, pqh, pet, pkt;
    Prefetch<64, TI> pv;
    Prefetch<64, float> pw;
    float n1[16], n2[16];   // rows 16 ty + li of N1, N2: this lane's MFMA A operands
    float pe = 0.f;
    auto wsof = [&](int c) { return ws + ((size_t)(base + c) * H + h) * G2Ws<D>::total; };
    auto fetch_next = [&](int c) {
        const long row0 = start + (long)c * BC;
        const int n = (int)min((long)BC, L - (long)c * BC);
        const float *Wc = wsof(c);
        pf1.fetch(Wc + G2Ws<D>::oF1, D, BC, tid);
        pqh.fetch(Wc + G2Ws<D>::oQH, D, BC, tid);
        pv.fetch(v + ((size_t)row0 * H + h) * D + dv0, (size_t)H * D, n, tid);
        pw.fetch(write + ((size_t)row0 * H + h) * D + dv0, (size_t)H * D, n, tid);
        if (tid < D) pe = Wc[G2Ws<D>::oEG + tid];
    };
    auto fetch_late = [&](int c) {
        const float *Wc = wsof(c);
        pet.fetch(Wc + G2Ws<D>::oET, D, BC, tid);
        pkt.fetch(Wc + G2Ws<D>::oKT, D, BC, tid);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            n1[m] = Wc[G2Ws<D>::oN1 + (16 * ty + li) * BC + 4 * m + lq];
            n2[m] = Wc[G2Ws<D>::oN2 + (16 * ty + li) * BC + 4 * m + lq];
        }
    };
    if (N > 0) fetch_next(0);
    for (int c = 0; c < N; ++c) {
        const long row0 = start + (long)c * BC;
        const int n = (int)min((long)BC, L - (long)c * BC);
#pragma unroll
        for (int t = 0; t < NTC; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
                sS[row * LF + col] = st[t][j];
            }
        pf1.commit(sX1, LF, tid);
        pqh.commit(sX2, LF, tid);
        pv.commit(sZ, LDN, tid);   // V slice; times w below
        pw.commit(sX, LDN, tid);   // w slice (scratch until X is formed)
        if (tid < D) seg[tid] = pe;
        __syncthreads();
        for (int e = tid; e < BC * 64; e += 512) {
            const int r = e >> 6, cc = e & 63;
            sZ[r * LDN + cc] *= sX[r * LDN + cc];
        }
        fetch_late(c);
        if (c + 1 < N) fetch_next(c + 1);
        __syncthreads();
        // X = -(F1 S^T + N1 Z), O = Qh S^T + N2 Z (64 tokens x 64 slice columns)
        f32x4 xa[2], oa[2];
        zero_n(xa);
        zero_n(oa);
        mm_rows2<D, 2>(sX1 + 16 * ty * LF, sX2 + 16 * ty * LF, LF, sS + 16 * tx0 * LF, LF, xa, oa,
                       lane);
#pragma unroll
        for (int m = 0; m < 16; ++m)
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const float zb = sZ[(4 * m + lq) * LDN + 16 * (tx0 + x) + li];
                xa[x] = mfma_f32(n1[m], zb, xa[x]);
                oa[x] = mfma_f32(n2[m], zb, oa[x]);
            }
        __syncthreads();   // F1, Qh and the w scratch consumed
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * ty + 4 * lq + j, col = 16 * (tx0 + x) + li;
                sX[r * LDN + col] = -xa[x][j];
                if (r < n) o[((size_t)(row0 + r) * H + h) * D + dv0 + col] = cvt<TO>(oa[x][j]);
            }
        pet.commit(sX1, LF, tid);
        pkt.commit(sX2, LF, tid);
        __syncthreads();
        // S <- S Diag(e^{G_n}) + X^T (E o e^{G_n - G}) + Z^T (K o e^{G_n - G})
#pragma unroll
        for (int t = 0; t < NTC; ++t) st[t] = st[t] * seg[16 * (tc0 + t) + li];
        mmn<BC, NTC>(sX + 16 * tr, 1, LDN, sX1 + 16 * tc0, LF, 1, 16, st, lane);
        mmn<BC, NTC>(sZ + 16 * tr, 1, LDN, sX2 + 16 * tc0, LF, 1, 16, st, lane);
        __syncthreads();
    }
    if (S_T) {
#pragma unroll
        for (int t = 0; t < NTC; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
                S_T[((size_t)uh * D + dv0 + row) * D + col] = st[t][j];
            }
    }
}

template <int D, typename TI, typename TO>
hipError_t launch_gdn2_t(int units, int T, int H, const int32_t *cu, const void *q,
                         const void *k, const void *v, const float *la, const float *erase,
                         const float *write, const float *S0, void *o, float *S_T, float *ws,
                         long nslots, hipStream_t st) {
    const int varlen = cu != nullptr;
    const int NC = varlen ? 0 : (T + BC - 1) / BC;
    const size_t nch = (size_t)nslots * H;
    if (nch > 0)
        hipLaunchKernelGGL((gdn2_prep_kernel<D, TI>), dim3((unsigned)std::min<size_t>(nch, 256)),
                           dim3(512), 0, st, T, H, units, NC, varlen, cu, (const TI *)q,
                           (const TI *)k, la, erase, ws, (int)nch);
    hipLaunchKernelGGL((gdn2_fwd_kernel<D, TI, TO>), dim3((unsigned)((long)units * H * (D / 64))),
                       dim3(512), 0, st, T, H, NC, varlen, cu, (const TI *)v, write, S0, ws,
                       (TO *)o, S_T);
    return hipGetLastError();
}

}  // namespace

bool gdn2_supported(int dk, int dv, int chunk, bool io_bf16) {
    if (chunk != BC || dk != dv) return false;
    return io_bf16 ? (dk == 64 || dk == 128) : dk == 64;
}

size_t gdn2_ws_bytes(int units, int T, int H, int d, bool varlen) {
    const long nslots = varlen ? (long)T / BC + units + 1 : (long)units * ((T + BC - 1) / BC);
    const size_t per = d == 128 ? G2Ws<128>::total : G2Ws<64>::total;
    return sizeof(float) * (size_t)nslots * H * per;
}

hipError_t launch_gdn2_fwd(int units, int T, int H, int d, bool io_bf16, bool o_bf16,
                           const int32_t *cu, const void *q, const void *k, const void *v,
                           const float *la, const float *erase, const float *write,
                           const float *S0, void *o, float *S_T, void *ws, hipStream_t st) {
    const long nslots = cu ? (long)T / BC + units + 1 : (long)units * ((T + BC - 1) / BC);
    float *w = (float *)ws;
#define GDN_G2(DV, TI, TO)                                                                    \
    return launch_gdn2_t<DV, TI, TO>(units, T, H, cu, q, k, v, la, erase, write, S0, o, S_T, w, \
                                     nslots, st)
    if (io_bf16) {
        if (d == 128) { if (o_bf16) GDN_G2(128, bf16, bf16); GDN_G2(128, bf16, float); }
        if (d == 64) { if (o_bf16) GDN_G2(64, bf16, bf16); GDN_G2(64, bf16, float); }
    } else if (d == 64) {
        if (o_bf16) GDN_G2(64, float, bf16);
        GDN_G2(64, float, float);
    }
#undef GDN_G2
    return hipErrorInvalidValue;
}

}  // namespace gdn
