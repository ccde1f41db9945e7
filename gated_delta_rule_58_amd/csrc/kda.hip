// Chunkwise forward of the delta rule with channel-wise decay (KDA) on
// gfx950, fp32 MFMA.
//
// "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
// (abstract) describes Kimi Delta Attention as the delta rule with
// channel-wise decay, reducing to Gated DeltaNet when the decay is a scalar;
// the pages print no equation.  The rule computed here lets the decay act on
// the key channels (columns of S) before the delta update:
//
//   S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
//   o_t = S_t q_t,   alpha_t in (0,1]^{d_k} given as log alpha_t.
//
// Chunk form (the WY/UT steps of the scalar rule with Diag(e^{G_r - G_i})
// inside the key products; G_r = sum_{s<=r} log alpha_s per channel):
//   A[r,i] = beta_r sum_c k_rc k_ic e^{G_rc - G_ic} (i < r),  T = (I + A)^{-1}
//   P[r,i] = sum_c q_rc k_ic e^{G_rc - G_ic}       (i <= r)
//   Delta  = T diag(beta) (V - (K o e^G) S^T)
//   O      = (Q o e^G) S^T + P Delta
//   S'     = S Diag(e^{G_n}) + Delta^T (K o e^{G_n - G})
//
// Two launches:
//   1. kda_prep (one workgroup per chunk and head): G, then A and P -- the
//      blocks below the diagonal as MFMA products of operands rescaled to a
//      reference token between the two blocks (every factor e^{<= 0}), the
//      diagonal blocks term by term -- T by the blocked inverse, and the
//      rescaled K o e^G, Q o e^G, K o e^{G_n - G}, e^{G_n};
//   2. kda_fwd (one workgroup per sequence, head and 64-column d_v slice,
//      chunks in order): the state recurrence and the outputs.
#include "fp32_tiles.h"

#include <mutex>

namespace gdn {
namespace {

using namespace tiles;


// Workspace block sizes (floats) per chunk and head.
template <int D> struct KdaWs {
    static constexpr size_t T = BC * BC, P = BC * BC, KG = BC * D, QG = BC * D, KT = BC * D,
                            EG = D, BETA = BC;
    static constexpr size_t total = T + P + KG + QG + KT + EG + BETA;
};

// ---------------------------------------------------------------- 1. prep
template <int D, typename TI>
__global__ __launch_bounds__(512) void kda_prep_kernel(
    int T, int H, int units, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ q, const TI *__restrict__ k, const float *__restrict__ la,
    const float *__restrict__ beta, float *__restrict__ ws) {
    constexpr int LI = ldx<TI, D>(), LF = D + 4;
    // K, Q and G, then A over G and T over Q once those are consumed (68 KB
    // for d = 128, so two workgroups share a CU)
    constexpr int BK = BC * LI * sizeof(TI), BNN = BC * LDN * 4;
    constexpr int BQ = BK > BNN ? BK : BNN, BG = BC * LF * 4 > BNN ? BC * LF * 4 : BNN;
    __shared__ __attribute__((aligned(16))) unsigned char smem[BK + BQ + BG];
    TI *sK = reinterpret_cast<TI *>(smem), *sQ = reinterpret_cast<TI *>(smem + BK);
    float *sG = reinterpret_cast<float *>(smem + BK + BQ);
    float *sA = sG, *sX = reinterpret_cast<float *>(smem + BK);
    __shared__ float sb[BC];
    const int slot = blockIdx.x / H, h = blockIdx.x % H;
    long row0;
    int n;
    if (!slot_chunk(slot, units, T, NC, varlen, cu, row0, n)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    float *W = ws + (size_t)blockIdx.x * KdaWs<D>::total;
    float *wT = W, *wP = wT + KdaWs<D>::T, *wKG = wP + KdaWs<D>::P, *wQG = wKG + KdaWs<D>::KG;
    float *wKT = wQG + KdaWs<D>::QG, *wEG = wKT + KdaWs<D>::KT, *wB = wEG + KdaWs<D>::EG;
    load_rows<D>(sK, LI, k, row0, n, H, h, 0, D, tid, 512);
    load_rows<D>(sQ, LI, q, row0, n, H, h, 0, D, tid, 512);
    load_rows<D>(sG, LF, la, row0, n, H, h, 0, D, tid, 512);
    if (tid < BC) {
        const float b = tid < n ? beta[(size_t)(row0 + tid) * H + h] : 0.f;
        sb[tid] = b;
        wB[tid] = b;
    }
    __syncthreads();
    if (tid < D) {   // prefix over the chunk per channel (padded rows add 0)
        float g = 0.f;
        for (int r = 0; r < BC; ++r) {
            g += sG[r * LF + tid];
            sG[r * LF + tid] = g;
        }
        wEG[tid] = expf(g);
    }
    __syncthreads();
    // rescaled operands for the sequential kernel
    for (int e = tid; e < BC * D / 4; e += 512) {
        const int r = e / (D / 4), c = (e % (D / 4)) * 4;
        const f32x4 g = *reinterpret_cast<const f32x4 *>(sG + r * LF + c);
        const f32x4 gn = *reinterpret_cast<const f32x4 *>(sG + (BC - 1) * LF + c);
        f32x4 kg, qg, kt;
        const f32x4 k4 = ld4f(sK + r * LI + c), q4 = ld4f(sQ + r * LI + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float kv = k4[j], qv = q4[j];
            const float eg = __expf(g[j]);
            kg[j] = kv * eg;
            qg[j] = qv * eg;
            kt[j] = kv * __expf(gn[j] - g[j]);
        }
        *reinterpret_cast<f32x4 *>(wKG + 4 * e) = kg;
        *reinterpret_cast<f32x4 *>(wQG + 4 * e) = qg;
        *reinterpret_cast<f32x4 *>(wKT + 4 * e) = kt;
    }
    // A and P, 16 x 16 blocks (br, bi), bi <= br: 10 blocks each.  The 8
    // diagonal blocks (one per wave) by diag_block; the 12 blocks below the
    // diagonal are MFMA products whose operands
    // are rescaled to the last token of block br - 1 (G_i >= G_ref >= G_r
    // channel by channel, so both factors are e^{<= 0}).
    f32x4 adiag, aoff = zero4();   // this wave's A entries (diagonal block; a block below,
                                   // waves 0-5: A's six blocks below are tasks 0-5)
    {
        const bool isP = wave >= 4;
        const int b = wave & 3;
        const TI *X = isP ? sQ : sK;
        const int i = 16 * b + li;
        const f32x4 acc = diag_block<D>(X, LI, sK, LI, sG, LF, b, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * b + 4 * lq + j;
            if (isP) wP[r * BC + i] = i <= r ? acc[j] : 0.f;
            adiag[j] = i < r ? sb[r] * acc[j] : 0.f;
        }
    }
    for (int task = wave; task < 12; task += 8) {
        const bool isP = task >= 6;
        int blk = isP ? task - 6 : task, br = 1;   // blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
        while (blk >= br) blk -= br++;
        const int bi = blk;
        const TI *X = isP ? sQ : sK;
        f32x4 acc = zero4();
        const float *gref = sG + (16 * br - 1) * LF;
        const int ra = 16 * br + li, rb = 16 * bi + li;
#pragma unroll 4
        for (int c0 = 0; c0 < D; c0 += 4) {
            const int c = c0 + lq;
            const float gr = gref[c];
            const float a = to_f32(X[ra * LI + c]) * __expf(sG[ra * LF + c] - gr);
            const float bb = to_f32(sK[rb * LI + c]) * __expf(gr - sG[rb * LF + c]);
            acc = mfma_f32(a, bb, acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * br + 4 * lq + j, ii = 16 * bi + li;
            if (isP) wP[r * BC + ii] = acc[j];
            if (!isP) aoff[j] = sb[r] * acc[j];
        }
    }
    // upper blocks of P are zero
    for (int e = tid; e < BC * BC; e += 512) {
        const int r = e >> 6, i = e & 63;
        if ((i >> 4) > (r >> 4)) wP[e] = 0.f;
    }
    __syncthreads();   // G, K, Q consumed: A goes over G, T over Q
    for (int e = tid; e < BC * LDN; e += 512) {
        sA[e] = 0.f;
        sX[e] = 0.f;
    }
    __syncthreads();
    if (wave < 4) {
        const int b = wave;
#pragma unroll
        for (int j = 0; j < 4; ++j) sA[(16 * b + 4 * lq + j) * LDN + 16 * b + li] = adiag[j];
    }
    if (wave < 6) {
        int blk = wave, br = 1;
        while (blk >= br) blk -= br++;
#pragma unroll
        for (int j = 0; j < 4; ++j) sA[(16 * br + 4 * lq + j) * LDN + 16 * blk + li] = aoff[j];
    }
    __syncthreads();
    block_inverse64(sA, sX, wave, lane);
    for (int e = tid; e < BC * BC / 4; e += 512)
        *reinterpret_cast<f32x4 *>(wT + 4 * e) =
            *reinterpret_cast<const f32x4 *>(sX + (e >> 4) * LDN + (e & 15) * 4);
}

// ---------------------------------------------------------------- 2. fwd
template <int D, typename TI, typename TO>
__global__ __launch_bounds__(512) void kda_fwd_kernel(
    int T, int H, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ v, const float *__restrict__ S0, const float *__restrict__ ws,
    TO *__restrict__ o, float *__restrict__ S_T) {
    constexpr int LF = D + 4, NTC = D / 32, NSL = D / 64;
    __shared__ __attribute__((aligned(16))) float sX1[BC * LF];   // K o e^G, then K o e^{G_n - G}
    __shared__ __attribute__((aligned(16))) float sX2[BC * LF];   // Q o e^G
    __shared__ __attribute__((aligned(16))) float sS[BC * LF];    // state slice: d_v rows x d_k
    __shared__ __attribute__((aligned(16))) float sT[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sZ[BC * LDN];   // V slice, then Z
    __shared__ __attribute__((aligned(16))) float sD[BC * LDN];   // Delta
    __shared__ float sb[BC], seg[D];
    const int uh = blockIdx.x / NSL, dv0 = 64 * (blockIdx.x % NSL);
    const int u = uh / H, h = uh % H;
    long start, L;
    unit_span(u, T, varlen, cu, start, L);
    const int N = (int)((L + BC - 1) / BC);
    const int base = unit_base(u, NC, varlen, cu);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int tr = wave & 3, tc0 = (wave >> 2) * NTC;   // state tiles
    const int ty = wave & 3, tx0 = 2 * (wave >> 2);     // 64 x 64 tiles
    f32x4 st[NTC];   // st[t][j] = S[dv0 + 16 tr + 4 lq + j][16 (tc0 + t) + li]
#pragma unroll
    for (int t = 0; t < NTC; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
            st[t][j] = S0 ? S0[((size_t)uh * D + dv0 + row) * D + col] : 0.f;
        }
    Prefetch<D, float> pkg, pqg, pkt;
    Prefetch<BC, float> pt;
    Prefetch<64, TI> pv;
    float pP[16];   // P[16 ty + li][4 m + lq], this lane's operand of P Delta
    float pb = 0.f, pe0 = 0.f;
    auto wsof = [&](int c) { return ws + ((size_t)(base + c) * H + h) * KdaWs<D>::total; };
    auto fetch_next = [&](int c) {   // operands of chunk c used in its first phases
        const long row0 = start + (long)c * BC;
        const int n = (int)min((long)BC, L - (long)c * BC);
        const float *W = wsof(c);
        pt.fetch(W, BC, BC, tid);
        pkg.fetch(W + KdaWs<D>::T + KdaWs<D>::P, D, BC, tid);
        pqg.fetch(W + KdaWs<D>::T + KdaWs<D>::P + KdaWs<D>::KG, D, BC, tid);
        pv.fetch(v + ((size_t)row0 * H + h) * D + dv0, (size_t)H * D, n, tid);
        const float *we = W + KdaWs<D>::T + KdaWs<D>::P + 3 * KdaWs<D>::KG;
        if (tid < BC) pb = we[D + tid];
        if (tid < D) pe0 = we[tid];
    };
    auto fetch_late = [&](int c) {   // operands of chunk c used in its last phases
        const float *W = wsof(c);
        pkt.fetch(W + KdaWs<D>::T + KdaWs<D>::P + 2 * KdaWs<D>::KG, D, BC, tid);
        const float *P = W + KdaWs<D>::T;
#pragma unroll
        for (int m = 0; m < 16; ++m) pP[m] = P[(16 * ty + li) * BC + 4 * m + lq];
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
        pt.commit(sT, LDN, tid);
        pkg.commit(sX1, LF, tid);
        pqg.commit(sX2, LF, tid);
        pv.commit(sZ, LDN, tid);
        if (tid < BC) sb[tid] = pb;
        if (tid < D) seg[tid] = pe0;
        __syncthreads();
        fetch_late(c);
        if (c + 1 < N) fetch_next(c + 1);
        // Z = diag(beta) (V - (K o e^G) S^T) in place of V; QS = (Q o e^G) S^T
        f32x4 y[2], qs[2];
        zero_n(y);
        zero_n(qs);
        mm_rows2<D, 2>(sX1 + 16 * ty * LF, sX2 + 16 * ty * LF, LF, sS + 16 * tx0 * LF, LF, y, qs,
                       lane);
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * ty + 4 * lq + j, col = 16 * (tx0 + x) + li;
                float *z = sZ + r * LDN + col;
                *z = sb[r] * (*z - y[x][j]);
            }
        __syncthreads();
        // Delta = T Z; K o e^{G_n - G} replaces K o e^G
        {
            f32x4 d[2];
            zero_n(d);
            mmn<BC, 2>(sT + 16 * ty * LDN, LDN, 1, sZ + 16 * tx0, LDN, 1, 16, d, lane);
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sD[(16 * ty + 4 * lq + j) * LDN + 16 * (tx0 + x) + li] = d[x][j];
        }
        pkt.commit(sX1, LF, tid);
        __syncthreads();
        // O = QS + P Delta (P from registers)
#pragma unroll
        for (int m = 0; m < 16; ++m)
#pragma unroll
            for (int x = 0; x < 2; ++x)
                qs[x] = mfma_f32(pP[m], sD[(4 * m + lq) * LDN + 16 * (tx0 + x) + li], qs[x]);
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * ty + 4 * lq + j, col = 16 * (tx0 + x) + li;
                if (r < n) o[((size_t)(row0 + r) * H + h) * D + dv0 + col] = cvt<TO>(qs[x][j]);
            }
        // S <- S Diag(e^{G_n}) + Delta^T (K o e^{G_n - G})
#pragma unroll
        for (int t = 0; t < NTC; ++t) st[t] = st[t] * seg[16 * (tc0 + t) + li];
        mmn<BC, NTC>(sD + 16 * tr, 1, LDN, sX1 + 16 * tc0, LF, 1, 16, st, lane);
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
hipError_t launch_kda_t(int units, int T, int H, const int32_t *cu, const void *q, const void *k,
                        const void *v, const float *la, const float *beta, const float *S0,
                        void *o, float *S_T, float *ws, long nslots, hipStream_t st) {
    const int varlen = cu != nullptr;
    const int NC = varlen ? 0 : (T + BC - 1) / BC;
    const size_t nch = (size_t)nslots * H;
    if (nch > 0)
        hipLaunchKernelGGL((kda_prep_kernel<D, TI>), dim3((unsigned)nch), dim3(512), 0, st, T, H,
                           units, NC, varlen, cu, (const TI *)q, (const TI *)k, la, beta, ws);
    hipLaunchKernelGGL((kda_fwd_kernel<D, TI, TO>), dim3((unsigned)((long)units * H * (D / 64))),
                       dim3(512), 0, st, T, H, NC, varlen, cu, (const TI *)v, S0, ws, (TO *)o,
                       S_T);
    return hipGetLastError();
}

}  // namespace

bool kda_supported(int dk, int dv, int chunk, bool io_bf16) {
    if (chunk != BC || dk != dv) return false;
    return io_bf16 ? (dk == 64 || dk == 128) : dk == 64;
}

size_t kda_ws_bytes(int units, int T, int H, int d, bool varlen) {
    const long nslots = varlen ? (long)T / BC + units + 1 : (long)units * ((T + BC - 1) / BC);
    const size_t per = d == 128 ? KdaWs<128>::total : KdaWs<64>::total;
    return sizeof(float) * (size_t)nslots * H * per;
}

// ---------------------------------------------------------------- no allocation
// Workspace of gdn_kda_fwd_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never
// passes `scratch` itself (on the host it only names the symbol); it asks
// the runtime for this device's address once and keeps it per device.
constexpr size_t kKdaScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kKdaScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t kda_scratch_bytes() { return kKdaScratchBytes; }

hipError_t kda_scratch_ptr(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_kda_fwd(int units, int T, int H, int d, bool io_bf16, bool o_bf16,
                          const int32_t *cu, const void *q, const void *k, const void *v,
                          const float *la, const float *beta, const float *S0, void *o,
                          float *S_T, void *ws, hipStream_t st) {
    const long nslots = cu ? (long)T / BC + units + 1 : (long)units * ((T + BC - 1) / BC);
    float *w = (float *)ws;
#define GDN_KDA(DV, TI, TO) \
    return launch_kda_t<DV, TI, TO>(units, T, H, cu, q, k, v, la, beta, S0, o, S_T, w, nslots, st)
    if (io_bf16) {
        if (d == 128) { if (o_bf16) GDN_KDA(128, bf16, bf16); GDN_KDA(128, bf16, float); }
        if (d == 64) { if (o_bf16) GDN_KDA(64, bf16, bf16); GDN_KDA(64, bf16, float); }
    } else if (d == 64) {
        if (o_bf16) GDN_KDA(64, float, bf16);
        GDN_KDA(64, float, float);
    }
#undef GDN_KDA
    return hipErrorInvalidValue;
}

}  // namespace gdn
