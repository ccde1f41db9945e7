// Chunkwise forward of the delta rule with channel-wise decay (KDA) on
// gfx950.
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
//   1. kda_prep (one workgroup per chunk and head, fp32 arithmetic): G, then
//      A and P -- the blocks below the diagonal as fp32 MFMA products of
//      operands rescaled to a reference token between the two blocks (every
//      factor e^{<= 0}), the diagonal blocks term by term -- T by the blocked
//      inverse; it writes K o e^G, Q o e^G, T diag(beta), P,
//      (K o e^{G_n - G})^T and e^{G_n} as bf16 hi + lo pairs, laid out as the
//      second launch keeps them in LDS;
//   2. kda_fwd (one workgroup per sequence, head and 64-column d_v slice,
//      chunks in order): the state recurrence and the outputs, every product
//      on the bf16 MFMA as three piece products (about 2^-16 relative, so
//      fp32-accurate to the precision the parity bar asks), its operand
//      regions copied global -> LDS by four loader waves three phases ahead.
#include "fp32_tiles.h"
#include "img_tiles.h"

#include <mutex>

namespace gdn {
namespace {

using namespace tiles;
using namespace img;

constexpr float kLog2e = 1.4426950408889634f;
// 2^x by the hardware exponential (the prep keeps the gate prefix G in base-2
// units, log2 e times the natural prefix, so that each exponential is one
// v_exp_f32 of a difference)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }


// The operands of the sequential launch, per chunk and head, as bf16 hi + lo
// pairs: K o e^G, Q o e^G (64 x D each), T diag(beta), P (64 x 64 each),
// (K o e^{G_n - G})^T (D x 64) and e^{G_n} (D floats).  Each row's 32-wide
// column blocks are in the D-order the MFMA fragments read (img_tiles.h).
// In LDS (KdaLds, offsets in bf16 elements) rows are padded by 8 elements so
// that the fragment reads are free of bank conflicts, in four regions of
// whole KB -- K o e^G | Q o e^G, T diag(beta), P, (K o e^{G_n - G})^T with
// e^{G_n} -- that the sequential launch copies one after another.  In the
// workspace (KdaWs) the same rows are dense: the pads would be 9-12% of the
// bytes written and read back.
template <int D> struct KdaLds {
    static constexpr int LK = D + 8, LC = BC + 8;   // row strides of the 64 x D and x 64 blocks
    static constexpr size_t up(size_t x) { return (x + 511) / 512 * 512; }
    static constexpr size_t KG = 0,                         // K o e^G, 64 x D: hi, lo
                            QG = KG + 2 * BC * LK,          // Q o e^G, 64 x D: hi, lo
                            TB = up(QG + 2 * BC * LK),      // T diag(beta), 64 x 64: hi, lo
                            P = up(TB + 2 * BC * LC),       // P, 64 x 64: hi, lo
                            KT = up(P + 2 * BC * LC),       // (K o e^{G_n - G})^T, D x 64: hi, lo
                            EG = KT + 2 * D * LC,           // e^{G_n}: D floats
                            total = up(EG + 2 * D);
    static_assert(TB == QG + 2 * BC * LK && P == TB + 2 * BC * LC && KT == P + 2 * BC * LC,
                  "regions are contiguous");
};
template <int D> struct KdaWs {
    static constexpr size_t KG = 0, QG = KG + 2 * BC * D, TB = QG + 2 * BC * D,
                            P = TB + 2 * BC * BC, KT = P + 2 * BC * BC, EG = KT + 2 * D * BC,
                            total = EG + 2 * D;
    static_assert(total % 64 == 0, "chunk-head images start on 128-byte lines");
};

// ---------------------------------------------------------------- 1. prep
template <int D, typename TI>
__global__ __launch_bounds__(512) void kda_prep_kernel(
    int T, int H, int units, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ q, const TI *__restrict__ k, const float *__restrict__ la,
    const float *__restrict__ beta, bf16 *__restrict__ ws) {
    typedef KdaWs<D> WS;
    constexpr int LI = ldx<TI, D>(), LF = D + 4;
    // K, Q and G, then A over G and T over Q once those are consumed (68 KB
    // for d = 128, so two workgroups share a CU)
    constexpr int BK = BC * LI * sizeof(TI), BNN = BC * LDN * 4;
    constexpr int BQ = BK > BNN ? BK : BNN, BG = BC * LF * 4 > BNN ? BC * LF * 4 : BNN;
    __shared__ __attribute__((aligned(16))) unsigned char smem[BK + BQ + BG];
    TI *sK = reinterpret_cast<TI *>(smem), *sQ = reinterpret_cast<TI *>(smem + BK);
    float *sG = reinterpret_cast<float *>(smem + BK + BQ);
    float *sA = sG, *sX = reinterpret_cast<float *>(smem + BK);
    // P is gathered over K once that is consumed, when it fits, and written
    // row by row with the other 16-byte stores (written block by block it
    // leaves lines to be written more than once)
    constexpr bool kStageP = BK >= BC * LDN * 4;
    float *sP = reinterpret_cast<float *>(smem);
    __shared__ __attribute__((aligned(16))) float sb[BC];
    const int slot = blockIdx.x / H, h = blockIdx.x % H;
    long row0;
    int n;
    if (!slot_chunk(slot, units, T, NC, varlen, cu, row0, n)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    bf16 *W = ws + (size_t)blockIdx.x * WS::total;
    float *wEG = reinterpret_cast<float *>(W + WS::EG);
    {   // every load in flight before the first LDS store (a loop that stores
        // each load waits for the memory round trip of each in turn)
        const size_t g0 = (size_t)row0 * H * D + (size_t)h * D;
        Prefetch<D, TI> pk, pq;
        Prefetch<D, float> pg;
        pk.fetch(k + g0, (size_t)H * D, n, tid);
        pq.fetch(q + g0, (size_t)H * D, n, tid);
        pg.fetch(la + g0, (size_t)H * D, n, tid);
        const float bv = tid < n ? beta[(size_t)(row0 + tid) * H + h] : 0.f;
        pk.commit(sK, LI, tid);
        pq.commit(sQ, LI, tid);
        pg.commit(sG, LF, tid);
        if (tid < BC) sb[tid] = bv;
    }
    __syncthreads();
    if (tid < D) {   // prefix over the chunk per channel, base-2 units (padded rows add 0)
        float g = 0.f;
        for (int r = 0; r < BC; ++r) {
            g += sG[r * LF + tid] * kLog2e;
            sG[r * LF + tid] = g;
        }
        wEG[tid] = exp2f(g);
    }
    __syncthreads();
    // rescaled operands of the sequential launch, one D-order group of 8
    // (16-byte stores) per item: K o e^G and Q o e^G along rows,
    // (K o e^{G_n - G})^T along the tokens of one channel
    for (int e = tid; e < BC * D / 8; e += 512) {
        const int r = e / (D / 8), p = 8 * (e % (D / 8));   // stored positions p..p+7
        const int c0 = (p & ~31) + (p & 31) / 2, c1 = c0 + 16;   // columns c0..+3, c1..+3
        const f32x4 g0 = *reinterpret_cast<const f32x4 *>(sG + r * LF + c0);
        const f32x4 g1 = *reinterpret_cast<const f32x4 *>(sG + r * LF + c1);
        const f32x4 k0 = ld4f(sK + r * LI + c0), k1 = ld4f(sK + r * LI + c1);
        const f32x4 q0 = ld4f(sQ + r * LI + c0), q1 = ld4f(sQ + r * LI + c1);
        f32x4 kg0, kg1, qg0, qg1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e0 = exp2_fast(g0[j]), e1 = exp2_fast(g1[j]);
            kg0[j] = k0[j] * e0;
            qg0[j] = q0[j] * e0;
            kg1[j] = k1[j] * e1;
            qg1[j] = q1[j] * e1;
        }
        const int off = r * D + p;
        put_pair8(W + WS::KG + off, W + WS::KG + BC * D + off, kg0, kg1);
        put_pair8(W + WS::QG + off, W + WS::QG + BC * D + off, qg0, qg1);
    }
    // (K o e^{G_n - G})^T: an item is four channels of one run of 4 tokens
    // (half of a D-order group of 8; the two halves go to neighbouring lanes,
    // whose 8-byte stores are adjacent), read as one piece of each token's row
    for (int e = tid; e < (D / 4) * (BC / 4); e += 512) {
        const int half = e & 1, grp = e >> 1;
        const int c4 = 4 * (grp / (BC / 8)), p = 8 * (grp % (BC / 8));
        const int rt = (p & ~31) + (p & 31) / 2 + 16 * half;   // tokens rt..rt+3
        const f32x4 gn = *reinterpret_cast<const f32x4 *>(sG + (BC - 1) * LF + c4);
        f32x4 kv[4];   // [channel][token]
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x4 g = *reinterpret_cast<const f32x4 *>(sG + (rt + j) * LF + c4);
            const f32x4 kk = ld4f(sK + (rt + j) * LI + c4);
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) kv[ch][j] = kk[ch] * exp2_fast(gn[ch] - g[ch]);
        }
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            const int off = (c4 + ch) * BC + p + 4 * half;
            put_pair4(W + WS::KT + off, W + WS::KT + D * BC + off, kv[ch]);
        }
    }
    // blocks of P above the diagonal are zero
    if constexpr (!kStageP)
    for (int e = tid; e < BC * BC / 4; e += 512) {
        const int r = e >> 4, i = (e & 15) * 4;
        if ((i >> 4) > (r >> 4)) {
            const int off = r * BC + dpos(i);
            put_pair4(W + WS::P + off, W + WS::P + BC * BC + off, zero4());
        }
    }
    // A and P, 16 x 16 blocks (br, bi), bi <= br: 10 blocks each.  The 8
    // diagonal blocks (one per wave) by diag_block; the 12 blocks below the
    // diagonal are MFMA products whose operands
    // are rescaled to the last token of block br - 1 (G_i >= G_ref >= G_r
    // channel by channel, so both factors are e^{<= 0}).  P goes straight
    // to the workspace; A stays in registers until G is consumed.
    f32x4 adiag, aoff = zero4();   // this wave's A entries (diagonal block; a block below,
                                   // waves 0-5: A's six blocks below are tasks 0-5)
    f32x4 pdiag = zero4(), poff = zero4();   // and P entries (waves 4-7; tasks 6-11)
    {
        const bool isP = wave >= 4;
        const int b = wave & 3;
        const TI *X = isP ? sQ : sK;
        const int i = 16 * b + li;
        const f32x4 acc = diag_block<D, true>(X, LI, sK, LI, sG, LF, b, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * b + 4 * lq + j;
            if (isP) {
                if constexpr (kStageP) {
                    pdiag[j] = i <= r ? acc[j] : 0.f;
                } else {
                    const int off = r * BC + dpos(i);
                    put_pair1(W + WS::P + off, W + WS::P + BC * BC + off, i <= r ? acc[j] : 0.f);
                }
            }
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
        // step j of channel group c0: lane (li, lq) supplies channel
        // c0 + 4 lq + j, so it reads its four channels with one vector read.
        // A: lane holds rows 16 br + 4 lq + j of column 16 bi + li; P is
        // formed transposed, so a lane holds row 16 br + li, columns
        // 16 bi + 4 lq + j (four consecutive stored positions)
#pragma unroll 2
        for (int c0 = 0; c0 < D; c0 += 16) {
            const int cb = c0 + 4 * lq;
            const f32x4 gr = *reinterpret_cast<const f32x4 *>(gref + cb);
            const f32x4 ga = *reinterpret_cast<const f32x4 *>(sG + ra * LF + cb);
            const f32x4 gb = *reinterpret_cast<const f32x4 *>(sG + rb * LF + cb);
            const f32x4 xa = ld4f(X + ra * LI + cb), kb = ld4f(sK + rb * LI + cb);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = xa[j] * exp2_fast(ga[j] - gr[j]), bb = kb[j] * exp2_fast(gr[j] - gb[j]);
                acc = isP ? mfma_f32(bb, a, acc) : mfma_f32(a, bb, acc);
            }
        }
        if (isP) {
            if constexpr (kStageP) {
                poff = acc;
            } else {
                const int off = (16 * br + li) * BC + dpos(16 * bi + 4 * lq);
                put_pair4(W + WS::P + off, W + WS::P + BC * BC + off, acc);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) aoff[j] = sb[16 * br + 4 * lq + j] * acc[j];
        }
    }
    __syncthreads();   // G, K, Q consumed: A goes over G, T over Q
    // blocks above the diagonal of T and P (A's are never read; the rest of
    // each is written whole below)
    zero_upper(sX, tid);
    if constexpr (kStageP) zero_upper(sP, tid);
    __syncthreads();
    if constexpr (kStageP) {
        if (wave >= 4) {
            const int b = wave & 3;
#pragma unroll
            for (int j = 0; j < 4; ++j) sP[(16 * b + 4 * lq + j) * LDN + 16 * b + li] = pdiag[j];
        }
        const int task = wave < 4 ? wave + 8 : wave;
        if (task >= 6) {
            int blk = task - 6, br = 1;
            while (blk >= br) blk -= br++;
            *reinterpret_cast<f32x4 *>(sP + (16 * br + li) * LDN + 16 * blk + 4 * lq) = poff;
        }
    }
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
    for (int e = tid; e < BC * BC / 8; e += 512) {   // T diag(beta) (and P)
        const int r = e >> 3, p = 8 * (e & 7);
        const int i0 = (p & ~31) + (p & 31) / 2, i1 = i0 + 16;
        const f32x4 t0 = *reinterpret_cast<const f32x4 *>(sX + r * LDN + i0) *
                         *reinterpret_cast<const f32x4 *>(sb + i0);
        const f32x4 t1 = *reinterpret_cast<const f32x4 *>(sX + r * LDN + i1) *
                         *reinterpret_cast<const f32x4 *>(sb + i1);
        const int off = r * BC + p;
        put_pair8(W + WS::TB + off, W + WS::TB + BC * BC + off, t0, t1);
        if constexpr (kStageP)
            put_pair8(W + WS::P + off, W + WS::P + BC * BC + off,
                      *reinterpret_cast<const f32x4 *>(sP + r * LDN + i0),
                      *reinterpret_cast<const f32x4 *>(sP + r * LDN + i1));
    }
}

// ---------------------------------------------------------------- 2. fwd
// One workgroup per (sequence, head, 64 columns of d_v), chunks in order,
// four phases per chunk:
//   1. Y = (K o e^G) S^T and QS = (Q o e^G) S^T        (region 1)
//   2. Delta = T diag(beta) (V - Y)                      (region 2 and V)
//   3. O = QS + P Delta                                  (region 3)
//   4. S^T <- Diag(e^{G_n}) S^T + (K o e^{G_n - G})^T Delta   (region 4)
// Waves 0-3 copy each region of the next chunk into LDS with direct
// global-to-LDS loads as soon as the consumers are done with the current
// one (region 1 of chunk c + 1 during phase 2 of chunk c, and so on), and
// before each barrier wait only until the region the next phase reads has
// landed: every copy has three phases to arrive.  Waves 4-7 each own 16
// columns of d_v: S^T (d_k x 16, fp32) in accumulator tiles, every product
// on the bf16 MFMA as the three piece products hi*hi + lo*hi + hi*lo of
// hi + lo pairs.
template <int D, typename TI, typename TO>
__global__ __launch_bounds__(512, 1) void kda_fwd_kernel(
    int T, int H, int NC, int varlen, int xcd_map, const int32_t *__restrict__ cu,
    const TI *__restrict__ v, const float *__restrict__ S0, const bf16 *__restrict__ ws,
    TO *__restrict__ o, float *__restrict__ S_T) {
    typedef KdaLds<D> WS;   // the LDS layout (padded rows)
    typedef KdaWs<D> WD;    // the workspace layout (dense rows)
    constexpr int NSL = D / 64, NKS = D / 32, NCT = D / 16;
    constexpr int LK = WS::LK, LC = WS::LC;
    constexpr int VP = 16 / sizeof(TI);               // V elements per 16-byte piece
    constexpr int VROWS = 1024 / (64 * sizeof(TI));   // V rows per KB
    // KB per region, and the fewest 1 KB copies any loader wave issues for it
    constexpr int K1 = WS::TB / 512, K2 = (WS::P - WS::TB) / 512, K3 = (WS::KT - WS::P) / 512,
                  K4 = (WS::total - WS::KT) / 512;
    constexpr int C1 = K1 / 4, C2 = K2 / 4 + BC / VROWS / 4, C3 = K3 / 4, C4 = K4 / 4;
    static_assert(BC / VROWS % 4 == 0 && C1 + C2 + C3 + C4 < 64, "copy counts");
    __shared__ __attribute__((aligned(16))) bf16 sKQ[WS::TB];             // region 1
    __shared__ __attribute__((aligned(16))) bf16 sTB[WS::P - WS::TB];     // region 2
    __shared__ __attribute__((aligned(16))) bf16 sP[WS::KT - WS::P];      // region 3
    __shared__ __attribute__((aligned(16))) bf16 sKT[WS::total - WS::KT]; // region 4
    __shared__ __attribute__((aligned(16))) TI sV[BC * 64];               // V slice
    const bf16 *sKG = sKQ + WS::KG, *sQG = sKQ + WS::QG;
    const float *sEG = reinterpret_cast<const float *>(sKT + (WS::EG - WS::KT));

    // Workgroup -> (unit, head, d_v slice); with xcd_map the slices of one
    // (unit, head) land on the same XCD (workgroups are dealt to the 8 XCDs
    // round-robin) and share its L2.
    const int b = blockIdx.x;
    int uh, sl;
    if (xcd_map) {
        uh = (b & 7) + 8 * (b / (8 * NSL));
        sl = (b >> 3) % NSL;
    } else {
        uh = b / NSL;
        sl = b % NSL;
    }
    const int u = uh / H, h = uh % H, dv0 = 64 * sl;
    long start, L;
    unit_span(u, T, varlen, cu, start, L);
    const int N = (int)((L + BC - 1) / BC);
    const int base = unit_base(u, NC, varlen, cu);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lq = lane >> 4;
    auto wsof = [&](int c) { return ws + ((size_t)(base + c) * H + h) * WD::total; };

    // ---- loaders (waves 0-3): wave w copies the KB pieces w, w + 4, ... of
    // a region's LDS image, each lane's 16 bytes from the dense workspace
    auto copy_region = [&](auto reg, bf16 *dst, const bf16 *src, int kb) {
        typedef decltype(reg) RG;
        for (int i = wave; i < kb; i += 4)
            lds_dma16(reinterpret_cast<char *>(dst) + 1024 * i,
                      reinterpret_cast<const char *>(src) + 16 * RG::src_chunk(64 * i + lane));
    };
    auto copy_v = [&](int c) {   // rows past the chunk repeat its last token (their
                                 // T diag(beta) columns are zero)
        const long row0 = start + (long)c * BC;
        const int n = (int)min((long)BC, L - (long)c * BC);
        for (int i = wave; i < BC / VROWS; i += 4) {
            const int r = min(VROWS * i + lane / (64 / VROWS), n - 1);
            const TI *src = v + ((size_t)(row0 + r) * H + h) * D + dv0 + VP * (lane % (64 / VROWS));
            lds_dma16(sV + 1024 / sizeof(TI) * i, src);
        }
    };
    auto copy1 = [&](int c) { copy_region(PaddedRegion<4, BC, D, 0>{}, sKQ, wsof(c) + WD::KG, K1); };
    auto copy2 = [&](int c) {
        copy_region(PaddedRegion<2, BC, BC, 0>{}, sTB, wsof(c) + WD::TB, K2);
        copy_v(c);
    };
    auto copy3 = [&](int c) { copy_region(PaddedRegion<2, BC, BC, 0>{}, sP, wsof(c) + WD::P, K3); };
    auto copy4 = [&](int c) {
        copy_region(PaddedRegion<2, D, BC, D / 4>{}, sKT, wsof(c) + WD::KT, K4);   // with e^{G_n}
    };

    // A loader wave's barrier: its copies for the next phase are waited for
    // by count (wait_vm) beforehand, and nothing is moved across it; a full
    // __syncthreads would wait for every copy in flight.
    auto loader_barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    if (wave < 4) {
        // ---- loaders.  Copies in issue order: 1(0) 2(0) 3(0) 4(0) | per
        // chunk c: 1(c+1) in phase 2, 2(c+1) in phase 3, 3(c+1) in phase 4,
        // 4(c+1) in phase 1 of chunk c + 1.  Before each barrier a wave waits
        // until the region the next phase reads has landed: the copies issued
        // after it may still be in flight.
        if (N > 0) {
            copy1(0);
            copy2(0);
            copy3(0);
            copy4(0);
            wait_vm<C2 + C3 + C4>();   // region 1 of chunk 0
        }
        loader_barrier();
        for (int c = 0; c < N; ++c) {
            const bool more = c + 1 < N;
            if (c > 0) copy4(c);
            wait_vm<C3 + C4>();        // region 2 of chunk c
            loader_barrier();
            if (more) {
                copy1(c + 1);
                wait_vm<C4 + C1>();    // region 3 of chunk c
            } else {
                wait_vm<C4>();
            }
            loader_barrier();
            if (more) {
                copy2(c + 1);
                wait_vm<C1 + C2>();    // region 4 of chunk c
            } else {
                wait_vm<0>();
            }
            loader_barrier();
            if (more) {
                copy3(c + 1);
                wait_vm<C2 + C3>();    // region 1 of chunk c + 1
            }
            loader_barrier();
        }
        return;
    }

    // ---- consumers (waves 4-7): d_v columns dv0 + 16 cw + li
    const int cw = wave - 4;
    const int vcol = dv0 + 16 * cw + li;
    f32x4 st[NCT];   // st[t][j] = S^T[16 t + 4 lq + j][vcol]
#pragma unroll
    for (int t = 0; t < NCT; ++t)
        st[t] = S0 ? *reinterpret_cast<const f32x4 *>(S0 + ((size_t)uh * D + vcol) * D + 16 * t + 4 * lq)
                   : zero4();
    __syncthreads();
    for (int c = 0; c < N; ++c) {
        // ---- phase 1: Y = (K o e^G) S^T, QS = (Q o e^G) S^T
        f32x4 y[4], qs[4];
        {
            bf16x8 sh[NKS], sl_[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) split_op(st[2 * ks], st[2 * ks + 1], sh[ks], sl_[ks]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 yy = zero4(), a = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int off = (16 * rt + li) * LK + 32 * ks + 8 * lq;
                    const bf16x8 kh = ld8(sKG + off), kl = ld8(sKG + BC * LK + off);
                    const bf16x8 qh = ld8(sQG + off), ql = ld8(sQG + BC * LK + off);
                    yy = mfma32(kh, sh[ks], yy);
                    a = mfma32(qh, sh[ks], a);
                    yy = mfma32(kl, sh[ks], yy);
                    a = mfma32(ql, sh[ks], a);
                    yy = mfma32(kh, sl_[ks], yy);
                    a = mfma32(qh, sl_[ks], a);
                }
                y[rt] = yy;
                qs[rt] = a;
            }
        }
        __syncthreads();
        // ---- phase 2: Delta = T diag(beta) (V - Y)
        bf16x8 dh[2], dl[2];   // Delta as D-order B operands (tokens 0-31, 32-63)
        {
            f32x4 z[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 vv;
                if constexpr (sizeof(TI) == 2) {
                    const bf16x4 x = lds_read_tr(sV + (16 * rt + 4 * lq + (li >> 2)) * 64 + 16 * cw +
                                                 4 * (li & 3));
#pragma unroll
                    for (int j = 0; j < 4; ++j) vv[j] = (float)x[j];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) vv[j] = to_f32(sV[(16 * rt + 4 * lq + j) * 64 + 16 * cw + li]);
                }
                z[rt] = vv - y[rt];
            }
            bf16x8 zh[2], zl[2];
            split_op(z[0], z[1], zh[0], zl[0]);
            split_op(z[2], z[3], zh[1], zl[1]);
            f32x4 dd[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int off = (16 * rt + li) * LC + 32 * ks + 8 * lq;
                    const bf16x8 th = ld8(sTB + off), tl = ld8(sTB + BC * LC + off);
                    acc = mfma32(th, zh[ks], acc);
                    acc = mfma32(tl, zh[ks], acc);
                    acc = mfma32(th, zl[ks], acc);
                }
                dd[rt] = acc;
            }
            split_op(dd[0], dd[1], dh[0], dl[0]);
            split_op(dd[2], dd[3], dh[1], dl[1]);
        }
        __syncthreads();
        // ---- phase 3: O = QS + P Delta
        {
            const long row0 = start + (long)c * BC;
            const int n = (int)min((long)BC, L - (long)c * BC);
            const rsrc_t ro = rows_rsrc(o + ((size_t)row0 * H + h) * D + dv0 + 16 * cw,
                                        (uint32_t)n * H * D * (uint32_t)sizeof(TO));
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = qs[rt];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int off = (16 * rt + li) * LC + 32 * ks + 8 * lq;
                    const bf16x8 ph = ld8(sP + off), pl = ld8(sP + BC * LC + off);
                    acc = mfma32(ph, dh[ks], acc);
                    acc = mfma32(pl, dh[ks], acc);
                    acc = mfma32(ph, dl[ks], acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    rsrc_store(cvt<TO>(acc[j]), ro, (uint32_t)(r * H * D + li) * (uint32_t)sizeof(TO));
                }
            }
        }
        __syncthreads();
        // ---- phase 4: S^T <- Diag(e^{G_n}) S^T + (K o e^{G_n - G})^T Delta
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            f32x4 acc = st[t] * *reinterpret_cast<const f32x4 *>(sEG + 16 * t + 4 * lq);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int off = (16 * t + li) * LC + 32 * ks + 8 * lq;
                const bf16x8 kh = ld8(sKT + off), kl = ld8(sKT + D * LC + off);
                acc = mfma32(kh, dh[ks], acc);
                acc = mfma32(kl, dh[ks], acc);
                acc = mfma32(kh, dl[ks], acc);
            }
            st[t] = acc;
        }
        __syncthreads();
    }
    if (S_T) {
#pragma unroll
        for (int t = 0; t < NCT; ++t)
            *reinterpret_cast<f32x4 *>(S_T + ((size_t)uh * D + vcol) * D + 16 * t + 4 * lq) = st[t];
    }
}

template <int D, typename TI, typename TO>
hipError_t launch_kda_t(int units, int T, int H, const int32_t *cu, const void *q, const void *k,
                        const void *v, const float *la, const float *beta, const float *S0,
                        void *o, float *S_T, bf16 *ws, long nslots, hipStream_t st) {
    const int varlen = cu != nullptr;
    const int NC = varlen ? 0 : (T + BC - 1) / BC;
    const size_t nch = (size_t)nslots * H;
    if (nch > 0)
        hipLaunchKernelGGL((kda_prep_kernel<D, TI>), dim3((unsigned)nch), dim3(512), 0, st, T, H,
                           units, NC, varlen, cu, (const TI *)q, (const TI *)k, la, beta, ws);
    const long nuh = (long)units * H;
    const int xcd_map = nuh % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((kda_fwd_kernel<D, TI, TO>), dim3((unsigned)(nuh * (D / 64))), dim3(512),
                       0, st, T, H, NC, varlen, xcd_map, cu, (const TI *)v, S0, ws, (TO *)o, S_T);
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
    return sizeof(bf16) * (size_t)nslots * H * per;
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
    bf16 *w = (bf16 *)ws;
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
