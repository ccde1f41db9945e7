// Gated DeltaNet-2 forward on gfx950: channel-wise decay with a
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
// state update.  The prep works in fp32 (fp32 MFMA); the sequential launch
// multiplies operand images the prep writes as bf16 hi + lo pairs on the
// bf16 MFMA (img_tiles.h).
#include "fp32_tiles.h"
#include "img_tiles.h"

namespace gdn {
namespace {

using namespace tiles;
using namespace img;

constexpr float kLog2e = 1.4426950408889634f;
// 2^x by the hardware exponential (inputs here are differences of base-2
// prefixes, <= 0 or bounded by the decay-span limit)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }


// The operands of the sequential launch, per chunk and head, as bf16 hi + lo
// pairs: F1, Qh (64 x D each), (E o e^{G_n - G})^T with e^{G_n},
// (K o e^{G_n - G})^T (D x 64 each), and N1 with N2 (64 x 64 each).  Each
// row's 32-wide column blocks are in the D-order the MFMA fragments read
// (img_tiles.h).  In LDS (G2Lds, offsets in bf16 elements) rows are padded by
// 8 elements so that the fragment reads are free of bank conflicts, in five
// regions of whole KB in the order the sequential launch reads them.  In the
// workspace (G2Ws) the same rows are dense: the pads would be 9-12% of the
// bytes written and read back.
template <int D> struct G2Lds {
    static constexpr int LK = D + 8, LC = BC + 8;   // row strides of the 64 x D and x 64 blocks
    static constexpr size_t up(size_t x) { return (x + 511) / 512 * 512; }
    static constexpr size_t F1 = 0,                       // T_e (K o e^G): hi, lo
                            QH = up(2 * BC * LK),         // Q o e^G - M (K o e^G): hi, lo
                            ET = QH + up(2 * BC * LK),    // (E o e^{G_n - G})^T: hi, lo
                            EG = ET + 2 * D * LC,         // e^{G_n}: D floats
                            KT = up(EG + 2 * D),          // (K o e^{G_n - G})^T: hi, lo
                            N1 = KT + up(2 * D * LC),     // T_e A_k: hi, lo
                            N2 = N1 + 2 * BC * LC,        // P_k - M A_k: hi, lo
                            total = up(N2 + 2 * BC * LC);
    static_assert(QH == 2 * BC * LK && KT - (EG + 2 * D) < 512 && N1 == KT + 2 * D * LC &&
                      total == N2 + 2 * BC * LC,
                  "regions are contiguous");
};
template <int D> struct G2Ws {
    static constexpr size_t F1 = 0, QH = F1 + 2 * BC * D, ET = QH + 2 * BC * D,
                            EG = ET + 2 * D * BC, KT = EG + 2 * D, N1 = KT + 2 * D * BC,
                            N2 = N1 + 2 * BC * BC, total = N2 + 2 * BC * BC;
    static_assert(total % 64 == 0, "chunk-head images start on 128-byte lines");
};

// ---------------------------------------------------------------- 1. prep
template <int D, typename TI>
__global__ __launch_bounds__(512) void gdn2_prep_kernel(
    int T, int H, int units, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ q, const TI *__restrict__ k, const float *__restrict__ la,
    const float *__restrict__ erase, bf16 *__restrict__ ws, int nch) {
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
    typedef G2Ws<D> WS;
    bf16 *W = ws + (size_t)ci * WS::total;
    float *wEG = reinterpret_cast<float *>(W + WS::EG);
    pk.commit(sK, LI, tid);
    pq.commit(sQ, LI, tid);
    pg.commit(sG, LF, tid);
    pe.commit(sE, LE, tid);
    zero_upper(sTe, tid);   // the inverse writes the rest of T_e
    __syncthreads();
    {   // prefix over the chunk per channel (padded rows add 0)
        // G is kept in base-2 units (log2 e times the natural prefix), so that
        // every exponential below is one v_exp_f32 of a difference
        const float gn = column_prefix<D>(sG, LF, tid, kLog2e);
        if (tid % (512 / D) == 0) wEG[tid / (512 / D)] = exp2f(gn);
    }
    for (int e = tid; e < BC * D / 4; e += 512) {   // E = b o k
        const int r = e / (D / 4), c = (e % (D / 4)) * 4;
        const f32x4 kv = ld4f(sK + r * LI + c);
        f32x4 *pe = reinterpret_cast<f32x4 *>(sE + r * LE + c);
        *pe = *pe * kv;
    }
    __syncthreads();
    // (E o e^{G_n - G})^T and (K o e^{G_n - G})^T for the state update, one
    // D-order group of 8 tokens of one channel per item (16-byte stores)
    for (int e = tid; e < D * BC / 8; e += 512) {
        const int c = e / (BC / 8), p = 8 * (e % (BC / 8));
        const int r0 = (p & ~31) + (p & 31) / 2, r1 = r0 + 16;   // tokens r0..+3, r1..+3
        const float gn = sG[(BC - 1) * LF + c];
        f32x4 e0, e1, k0, k1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float t0 = exp2_fast(gn - sG[(r0 + j) * LF + c]), t1 = exp2_fast(gn - sG[(r1 + j) * LF + c]);
            e0[j] = sE[(r0 + j) * LE + c] * t0;
            e1[j] = sE[(r1 + j) * LE + c] * t1;
            k0[j] = to_f32(sK[(r0 + j) * LI + c]) * t0;
            k1[j] = to_f32(sK[(r1 + j) * LI + c]) * t1;
        }
        const int off = c * BC + p;
        put_pair8(W + WS::ET + off, W + WS::ET + D * BC + off, e0, e1);
        put_pair8(W + WS::KT + off, W + WS::KT + D * BC + off, k0, k1);
    }
    // The four channel-weighted products, 16 x 16 blocks (br, bi), bi <= br:
    // matrix mx = 0 A_e (rows K, columns E), 1 A_k (K, K), 2 P_e (Q, E),
    // 3 P_k (Q, K).  Each block is one MFMA product of operands rescaled to
    // the prefix just before block br (the last token of block br - 1, or 0):
    // every factor is e^{<= 0} below the diagonal, and on it too unless the
    // block's decay span exceeds 60, when the block is formed term by term
    // instead.  The four matrices of one block share both factors, so wave w
    // forms all four of block w (blocks numbered row by row: (0,0) (1,0)
    // (1,1) (2,0) ...) -- two exponentials per channel step for four
    // products -- and one matrix of block 8 or 9, five interleaved chains in
    // all.
    int cn;
    f32x4 res[5];   // res[mx]: block w, matrix mx; res[4]: block 8 + w / 4, matrix w % 4
    auto blk_of = [](int e, int &br, int &bi) {
        int blk = e, r = 0;
        while (blk > r) blk -= ++r;
        br = r;
        bi = blk;
    };
    int bmr, bmi, bxr, bxi;
    blk_of(wave, bmr, bmi);
    blk_of(8 + (wave >> 2), bxr, bxi);
    const int mxx = wave & 3;
    {
        const int ram = 16 * bmr + li, rbm = 16 * bmi + li, grm = bmr > 0 ? 16 * bmr - 1 : 0;
        const float gonm = bmr > 0 ? 1.f : 0.f;   // reference prefix 0 for the first block row
        const int rax = 16 * bxr + li, rbx = 16 * bxi + li, grx = 16 * bxr - 1;
        const bool termsm = bmi == bmr && diag_span<D>(sG, LF, bmr, lane) > 60.f * kLog2e;
        const bool termsx = bxi == bxr && diag_span<D>(sG, LF, bxr, lane) > 60.f * kLog2e;
        const TI *Xx = mxx < 2 ? sK : sQ;   // the extra chain's rows
        const bool colE = (mxx & 1) == 0;   // and its columns: E (A_e, P_e) or K
#pragma unroll
        for (int s = 0; s < 5; ++s) res[s] = zero4();
        // Step j of channel group c0 gives lane (li, lq) the k slot of
        // channel c0 + 4 lq + j (both operands alike), so a lane reads its
        // four channels of a row with one 16-byte (fp32) or 8-byte (bf16) read.
#pragma unroll 2
        for (int c0 = 0; c0 < D; c0 += 16) {
            const int cb = c0 + 4 * lq;
            const f32x4 gr4 = *reinterpret_cast<const f32x4 *>(sG + grm * LF + cb) * gonm;
            const f32x4 ga = *reinterpret_cast<const f32x4 *>(sG + ram * LF + cb);
            const f32x4 gb = *reinterpret_cast<const f32x4 *>(sG + rbm * LF + cb);
            const f32x4 ka = ld4f(sK + ram * LI + cb), qa = ld4f(sQ + ram * LI + cb);
            const f32x4 eb4 = *reinterpret_cast<const f32x4 *>(sE + rbm * LE + cb);
            const f32x4 kb = ld4f(sK + rbm * LI + cb);
            const f32x4 gx4 = *reinterpret_cast<const f32x4 *>(sG + grx * LF + cb);
            const f32x4 xa = ld4f(Xx + rax * LI + cb);
            const f32x4 gxa = *reinterpret_cast<const f32x4 *>(sG + rax * LF + cb);
            const f32x4 yb =
                colE ? *reinterpret_cast<const f32x4 *>(sE + rbx * LE + cb) : ld4f(sK + rbx * LI + cb);
            const f32x4 gxb = *reinterpret_cast<const f32x4 *>(sG + rbx * LF + cb);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ea = exp2_fast(ga[j] - gr4[j]), eb = exp2_fast(gr4[j] - gb[j]);
                const float ak = ka[j] * ea, aq = qa[j] * ea, be = eb4[j] * eb, bk = kb[j] * eb;
                res[0] = mfma_f32(ak, be, res[0]);
                res[1] = mfma_f32(ak, bk, res[1]);
                res[2] = mfma_f32(aq, be, res[2]);
                res[3] = mfma_f32(aq, bk, res[3]);
                res[4] = mfma_f32(xa[j] * exp2_fast(gxa[j] - gx4[j]), yb[j] * exp2_fast(gx4[j] - gxb[j]), res[4]);
            }
        }
        if (termsm) {
            res[0] = diag_terms<D, true>(sK, LI, sE, LE, sG, LF, bmr, lane);
            res[1] = diag_terms<D, true>(sK, LI, sK, LI, sG, LF, bmr, lane);
            res[2] = diag_terms<D, true>(sQ, LI, sE, LE, sG, LF, bmr, lane);
            res[3] = diag_terms<D, true>(sQ, LI, sK, LI, sG, LF, bmr, lane);
        }
        if (termsx)
            res[4] = colE ? diag_terms<D, true>(Xx, LI, sE, LE, sG, LF, bxr, lane)
                          : diag_terms<D, true>(Xx, LI, sK, LI, sG, LF, bxr, lane);
        // the next pair's inputs: issued here, where the waves of the
        // lighter block products would wait at the barrier anyway, rather
        // than all at once at the top of the pair
        cn = next(ci + gridDim.x);
        // keep strict (A) or inclusive (P) lower entries
#pragma unroll
        for (int s = 0; s < 5; ++s) {
            const int mx = s < 4 ? s : mxx, br = s < 4 ? bmr : bxr, bi = s < 4 ? bmi : bxi;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * br + 4 * lq + j, i = 16 * bi + li;
                if (mx < 2 ? i >= r : i > r) res[s][j] = 0.f;
            }
        }
    }
    __syncthreads();   // E consumed: A_e and A_k go over it
    // blocks above the diagonal of A_k, P_e, P_k, and of A_e (never read by
    // the inverse; M, stored over A_e, is lower triangular)
    zero_upper(sAe, tid);
    zero_upper(sAk, tid);
    zero_upper(sPe, tid);
    zero_upper(sPk, tid);
    for (int e = tid; e < BC * D / 4; e += 512) {   // G -> e^G: only F1 and Qh read it from here on
        f32x4 *pg = reinterpret_cast<f32x4 *>(sG + (e / (D / 4)) * LF + (e % (D / 4)) * 4);
        f32x4 x = *pg;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = exp2_fast(x[j]);
        *pg = x;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 5; ++s) {
        const int mx = s < 4 ? s : mxx, br = s < 4 ? bmr : bxr, bi = s < 4 ? bmi : bxi;
        float *dst = mx == 0 ? sAe : mx == 1 ? sAk : mx == 2 ? sPe : sPk;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[(16 * br + 4 * lq + j) * LDN + 16 * bi + li] = res[s][j];
    }
    __syncthreads();
    block_inverse64(sAe, sTe, wave, lane);   // T_e (ends with a barrier)
    // The folds multiply lower triangular 64 x 64 factors (T_e, P_e, P_k, M
    // lower, A_k strictly lower), so 16 x 16 output block (rb, cb) of M, N1
    // and N2 is zero above the diagonal and sums only over the k blocks
    // cb..rb, and row block rb of F1 and Qh over the k blocks 0..rb.  The
    // blocks are dealt to the waves so that each forms about as many block
    // products.
    // tile (rb, cb) of X Y, k blocks cb..rb (X, Y 64 x 64 in LDS, row stride LDN)
    auto tile_mm = [&](const float *X, const float *Y, int rb, int cb) {
        f32x4 acc[1];
        zero_n(acc);
        for (int kb = cb; kb <= rb; ++kb)
            mmn<16, 1>(X + 16 * rb * LDN + 16 * kb, LDN, 1, Y + 16 * kb * LDN + 16 * cb, LDN, 1, 0, acc, lane);
        return acc[0];
    };
    // the same block transposed: lane (i, q) gets rows 16 rb + i, columns
    // 16 cb + 4 q .. + 3 of X Y (four consecutive columns of one row)
    auto tile_mm_t = [&](const float *X, const float *Y, int rb, int cb) {
        f32x4 acc[1];
        zero_n(acc);
        for (int kb = cb; kb <= rb; ++kb)
            mmn<16, 1>(Y + 16 * kb * LDN + 16 * cb, 1, LDN, X + 16 * rb * LDN + 16 * kb, 1, LDN, 0, acc, lane);
        return acc[0];
    };
    // a zero block of a 64 x 64 image (rows 16 rb.., columns 16 cb..), 8-byte stores
    auto zero_img = [&](bf16 *img, int rb, int cb) {
        const int off = (16 * rb + li) * BC + dpos(16 * cb + 4 * lq);
        put_pair4(img + off, img + BC * BC + off, zero4());
    };
    // Block lists as 32-bit constants picked by the (wave-uniform) wave index,
    // so they stay in scalar registers: entry e in bits 4e..4e+3 encodes block
    // (rb, cb) as 4 rb + cb, the count is in bits 28-31.
    auto blist = [](unsigned n, unsigned a, unsigned b = 0, unsigned c = 0, unsigned d = 0) {
        return (n << 28) | a | (b << 4) | (c << 8) | (d << 12);
    };
    const int uw = __builtin_amdgcn_readfirstlane(wave);
    const int m = uw >> 1;
    const bool isN1 = uw & 1;
    const unsigned kMN = m == 0 ? blist(2, 12, 0) : m == 1 ? blist(2, 13, 4)
                       : m == 2 ? blist(2, 8, 14) : blist(4, 9, 5, 10, 15);
    const unsigned kN1z = m == 0 ? blist(2, 1, 2) : m == 1 ? blist(2, 3, 6)
                        : m == 2 ? blist(2, 7, 11) : 0u;
    const unsigned kN2 = uw == 0 ? blist(1, 12) : uw == 1 ? blist(1, 13) : uw == 2 ? blist(1, 8)
                       : uw == 3 ? blist(2, 9, 0) : uw == 4 ? blist(2, 14, 5)
                       : uw == 5 ? blist(2, 4, 10) : uw == 6 ? blist(1, 15) : 0u;
    const unsigned kN2z = uw == 1 ? blist(1, 1) : uw == 2 ? blist(1, 2) : uw == 3 ? blist(1, 3)
                        : uw == 4 ? blist(1, 6) : uw == 5 ? blist(1, 7) : uw == 6 ? blist(1, 11) : 0u;
    auto nblk = [](unsigned l) { return (int)(l >> 28); };
    auto blk = [](unsigned l, int e) { return (int)((l >> (4 * e)) & 15); };
    {   // M = P_e T_e (even waves, over A_e) and N1 = T_e A_k (odd waves, to the workspace)
        for (int e = 0; e < nblk(kMN); ++e) {
            const int rb = blk(kMN, e) >> 2, cb = blk(kMN, e) & 3;
            if (isN1) {
                const f32x4 acc = tile_mm_t(sTe, sAk, rb, cb);
                const int off = (16 * rb + li) * BC + dpos(16 * cb + 4 * lq);
                put_pair4(W + WS::N1 + off, W + WS::N1 + BC * BC + off, acc);
            } else {
                const f32x4 acc = tile_mm(sPe, sTe, rb, cb);
#pragma unroll
                for (int j = 0; j < 4; ++j) sAe[(16 * rb + 4 * lq + j) * LDN + 16 * cb + li] = acc[j];
            }
        }
        if (!isN1)
            for (int e = 0; e < nblk(kN1z); ++e) zero_img(W + WS::N1, blk(kN1z, e) >> 2, blk(kN1z, e) & 3);
    }
    __syncthreads();
    float *sM = sAe;
    // N2 = P_k - M A_k
    for (int e = 0; e < nblk(kN2); ++e) {
        const int rb = blk(kN2, e) >> 2, cb = blk(kN2, e) & 3;
        const f32x4 acc = tile_mm_t(sM, sAk, rb, cb);
        const int r = 16 * rb + li, c = 16 * cb + 4 * lq;
        const int off = r * BC + dpos(c);
        put_pair4(W + WS::N2 + off, W + WS::N2 + BC * BC + off,
                  *reinterpret_cast<const f32x4 *>(sPk + r * LDN + c) - acc);
    }
    for (int e = 0; e < nblk(kN2z); ++e) zero_img(W + WS::N2, blk(kN2z, e) >> 2, blk(kN2z, e) & 3);
    // F1 = T_e (K o e^G) and Qh = Q o e^G - M (K o e^G), with K o e^G formed
    // in the operand reads.  Wave w takes 16 columns (column tile ct) and
    // the row blocks in rbs: all four for d = 128; for d = 64 two waves share
    // a column tile, rows {3, 0} and {2, 1}.  Formed transposed, so that a
    // lane holds four consecutive columns of one row.
    {
        constexpr int NCT = D / 16, NRB = NCT == 8 ? 4 : 2;
        static_assert(NCT == 8 || NCT == 4, "d = 64 or 128");
        const int ct = wave % NCT;
        int rbs[NRB];
        if constexpr (NRB == 4) {
#pragma unroll
            for (int x = 0; x < 4; ++x) rbs[x] = x;
        } else {
            rbs[0] = wave < 4 ? 0 : 1;
            rbs[1] = wave < 4 ? 3 : 2;
        }
        f32x4 f1[NRB], qh[NRB];
        zero_n(f1);
        zero_n(qh);
        const int c = 16 * ct + li;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int kk = 0; kk < 16; kk += 4) {
                const int kr = 16 * kb + kk + lq;
                const float b = to_f32(sK[kr * LI + c]) * sG[kr * LF + c];
#pragma unroll
                for (int x = 0; x < NRB; ++x) {
                    if (rbs[x] < kb) continue;   // wave-uniform
                    const int rw = (16 * rbs[x] + li) * LDN + kr;
                    f1[x] = mfma_f32(b, sTe[rw], f1[x]);
                    qh[x] = mfma_f32(b, sM[rw], qh[x]);
                }
            }
        }
#pragma unroll
        for (int x = 0; x < NRB; ++x) {
            const int r = 16 * rbs[x] + li, c4 = 16 * ct + 4 * lq;   // columns c4..c4+3
            const f32x4 g = *reinterpret_cast<const f32x4 *>(sG + r * LF + c4);   // e^G
            const f32x4 qv = ld4f(sQ + r * LI + c4);
            f32x4 qg;
#pragma unroll
            for (int j = 0; j < 4; ++j) qg[j] = qv[j] * g[j] - qh[x][j];
            const int off = r * D + dpos(c4);
            put_pair4(W + WS::F1 + off, W + WS::F1 + BC * D + off, f1[x]);
            put_pair4(W + WS::QH + off, W + WS::QH + BC * D + off, qg);
        }
    }
    __syncthreads();   // every LDS operand consumed before the next pair's commit
    ci = cn;
    }
}

// ---------------------------------------------------------------- 2. fwd
// One workgroup per (sequence, head, 64 columns of d_v), chunks in order,
// five phases per chunk:
//   1. a = F1 S^T                                   (F1 in buffer U)
//   2. b = Qh S^T                                   (Qh in buffer W)
//   3. Z = w o v; X = -(a + N1 Z), O = b + N2 Z     (N1, N2, w, v)
//   4. S^T <- Diag(e^{G_n}) S^T + (E o e^{G_n - G})^T X   (buffer U)
//   5. S^T <- S^T + (K o e^{G_n - G})^T Z                  (buffer W)
// Waves 0-3 copy each region into LDS with direct global-to-LDS loads as
// soon as its buffer is free (buffer U takes (E o e^{G_n - G})^T during
// phase 2 and the next F1 during phase 5; buffer W takes (K o e^{G_n - G})^T
// during phase 3 and the next Qh during the next phase 1; N1, N2, w and v of
// the next chunk load during phase 4), and before each barrier wait by count
// for the region the next phase reads.  Waves 4-7 each own 16 columns of
// d_v: S^T (d_k x 16, fp32) in accumulator tiles, every product on the bf16
// MFMA as the three piece products of hi + lo pairs.
template <int D, typename TI, typename TO>
__global__ __launch_bounds__(512, 1) void gdn2_fwd_kernel(
    int T, int H, int NC, int varlen, int xcd_map, const int32_t *__restrict__ cu,
    const TI *__restrict__ v, const float *__restrict__ write, const float *__restrict__ S0,
    const bf16 *__restrict__ ws, TO *__restrict__ o, float *__restrict__ S_T) {
    typedef G2Lds<D> WS;   // the LDS layout (padded rows)
    typedef G2Ws<D> WD;    // the workspace layout (dense rows)
    constexpr int NSL = D / 64, NKS = D / 32, NCT = D / 16;
    constexpr int LK = WS::LK, LC = WS::LC;
    constexpr int VP = 16 / sizeof(TI);               // V elements per 16-byte piece
    constexpr int VROWS = 1024 / (64 * sizeof(TI));   // V rows per KB
    constexpr int WROWS = 4;                          // w (fp32) rows per KB
    // KB per region, and the fewest 1 KB copies any loader wave issues for it
    constexpr int KU1 = (WS::QH - WS::F1) / 512, KW1 = (WS::ET - WS::QH) / 512,
                  KU2 = (WS::KT - WS::ET) / 512, KW2 = (WS::N1 - WS::KT) / 512,
                  KR = (WS::total - WS::N1) / 512;
    constexpr int CU2 = KU2 / 4, CW1 = KW1 / 4, CW2 = KW2 / 4,
                  CR = KR / 4 + BC / WROWS / 4 + BC / VROWS / 4;
    static_assert(BC / VROWS % 4 == 0 && CU2 + CW2 + CR < 64, "copy counts");
    constexpr int BU = KU1 > KU2 ? KU1 : KU2, BW = KW1 > KW2 ? KW1 : KW2;
    __shared__ __attribute__((aligned(16))) bf16 sU[BU * 512];     // F1, then E^T and e^{G_n}
    __shared__ __attribute__((aligned(16))) bf16 sW[BW * 512];     // Qh, then K^T
    __shared__ __attribute__((aligned(16))) bf16 sN[KR * 512];     // N1, N2
    __shared__ __attribute__((aligned(16))) float sWg[BC * 64];    // write gate slice
    __shared__ __attribute__((aligned(16))) TI sV[BC * 64];        // V slice
    const float *sEG = reinterpret_cast<const float *>(sU + (WS::EG - WS::ET));

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

    if (wave < 4) {
        // ---- loaders: wave w copies the KB pieces w, w + 4, ... of a
        // region's LDS image, each lane's 16 bytes from the dense workspace
        auto copy_region = [&](auto reg, bf16 *dst, const bf16 *src, int kb) {
            typedef decltype(reg) RG;
            for (int i = wave; i < kb; i += 4)
                lds_dma16(reinterpret_cast<char *>(dst) + 1024 * i,
                          reinterpret_cast<const char *>(src) + 16 * RG::src_chunk(64 * i + lane));
        };
        typedef PaddedRegion<2, BC, D, 0> RgF;        // F1 or Qh
        typedef PaddedRegion<2, D, BC, D / 4> RgE;    // (E o e^{G_n - G})^T with e^{G_n}
        typedef PaddedRegion<2, D, BC, 0> RgK;        // (K o e^{G_n - G})^T
        typedef PaddedRegion<4, BC, BC, 0> RgN;       // N1, N2
        // v and w rows past the chunk repeat its last token: the columns of
        // N1, N2 and the rows of (K o e^{G_n - G})^T they meet are zero
        auto copy_r = [&](int c) {
            copy_region(RgN{}, sN, wsof(c) + WD::N1, KR);
            const long row0 = start + (long)c * BC;
            const int n = (int)min((long)BC, L - (long)c * BC);
            for (int i = wave; i < BC / VROWS; i += 4) {
                const int r = min(VROWS * i + lane / (64 / VROWS), n - 1);
                lds_dma16(sV + 1024 / sizeof(TI) * i,
                          v + ((size_t)(row0 + r) * H + h) * D + dv0 + VP * (lane % (64 / VROWS)));
            }
            for (int i = wave; i < BC / WROWS; i += 4) {
                const int r = min(WROWS * i + lane / 16, n - 1);
                lds_dma16(sWg + 256 * i, write + ((size_t)(row0 + r) * H + h) * D + dv0 + 4 * (lane % 16));
            }
        };
        auto loader_barrier = [&]() {   // the copies are waited for by count beforehand
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // Copies in issue order: U1(0) W1(0) R(0) | per chunk c: W1(c) (c > 0)
        // in phase 1, U2(c) in 2, W2(c) in 3, R(c+1) in 4, U1(c+1) in 5.
        if (N > 0) {
            copy_region(RgF{}, sU, wsof(0) + WD::F1, KU1);
            copy_region(RgF{}, sW, wsof(0) + WD::QH, KW1);
            copy_r(0);
            wait_vm<CW1 + CR>();   // F1 of chunk 0
        }
        loader_barrier();
        for (int c = 0; c < N; ++c) {
            const bool more = c + 1 < N;
            if (c > 0) copy_region(RgF{}, sW, wsof(c) + WD::QH, KW1);
            wait_vm<0>();          // Qh of chunk c (and N1, N2, w, v before it)
            loader_barrier();
            copy_region(RgE{}, sU, wsof(c) + WD::ET, KU2);
            wait_vm<CU2>();
            loader_barrier();
            copy_region(RgK{}, sW, wsof(c) + WD::KT, KW2);
            wait_vm<CW2>();        // E^T of chunk c
            loader_barrier();
            if (more) {
                copy_r(c + 1);
                wait_vm<CR>();     // K^T of chunk c
            } else {
                wait_vm<0>();
            }
            loader_barrier();
            if (more) {
                copy_region(RgF{}, sU, wsof(c + 1) + WD::F1, KU1);
                wait_vm<0>();      // F1 of chunk c + 1
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
    // A x S^T over 64 rows and d_k (A: hi at p, lo at p + lo_off; rows of lda)
    auto rows_st = [&](const bf16 *p, int lda, int lo_off, const bf16x8 (&sh)[NKS],
                       const bf16x8 (&sl)[NKS], f32x4 (&acc)[4]) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 a = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int off = (16 * rt + li) * lda + 32 * ks + 8 * lq;
                const bf16x8 xh = ld8(p + off), xl = ld8(p + lo_off + off);
                a = mfma32(xh, sh[ks], a);
                a = mfma32(xl, sh[ks], a);
                a = mfma32(xh, sl[ks], a);
            }
            acc[rt] = a;
        }
    };
    // acc[t] += A_t B over 64 tokens (A: rows 16 t + li at p, lo at + lo_off;
    // B: D-order pairs over tokens 0-31, 32-63)
    auto tok_prod = [&](const bf16 *p, int lo_off, const bf16x8 (&bh)[2], const bf16x8 (&bl)[2],
                        f32x4 &acc, int t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int off = (16 * t + li) * LC + 32 * ks + 8 * lq;
            const bf16x8 xh = ld8(p + off), xl = ld8(p + lo_off + off);
            acc = mfma32(xh, bh[ks], acc);
            acc = mfma32(xl, bh[ks], acc);
            acc = mfma32(xh, bl[ks], acc);
        }
    };
    for (int c = 0; c < N; ++c) {
        f32x4 a[4], bq[4];
        {
            bf16x8 sh[NKS], sl_[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) split_op(st[2 * ks], st[2 * ks + 1], sh[ks], sl_[ks]);
            rows_st(sU, LK, BC * LK, sh, sl_, a);     // phase 1: F1 S^T
            __syncthreads();
            rows_st(sW, LK, BC * LK, sh, sl_, bq);    // phase 2: Qh S^T
        }
        __syncthreads();
        // ---- phase 3: Z = w o v, X = -(F1 S^T + N1 Z), O = Qh S^T + N2 Z
        bf16x8 zh[2], zl[2], xh[2], xl[2];
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
#pragma unroll
                for (int j = 0; j < 4; ++j) z[rt][j] = vv[j] * sWg[(16 * rt + 4 * lq + j) * 64 + 16 * cw + li];
            }
            split_op(z[0], z[1], zh[0], zl[0]);
            split_op(z[2], z[3], zh[1], zl[1]);
            const long row0 = start + (long)c * BC;
            const int n = (int)min((long)BC, L - (long)c * BC);
            const rsrc_t ro = rows_rsrc(o + ((size_t)row0 * H + h) * D + dv0 + 16 * cw,
                                        (uint32_t)n * H * D * (uint32_t)sizeof(TO));
            f32x4 x[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 xa = a[rt], oa = bq[rt];
                tok_prod(sN, BC * LC, zh, zl, xa, rt);
                tok_prod(sN + 2 * BC * LC, BC * LC, zh, zl, oa, rt);
                x[rt] = -xa;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    rsrc_store(cvt<TO>(oa[j]), ro, (uint32_t)(r * H * D + li) * (uint32_t)sizeof(TO));
                }
            }
            split_op(x[0], x[1], xh[0], xl[0]);
            split_op(x[2], x[3], xh[1], xl[1]);
        }
        __syncthreads();
        // ---- phase 4: S^T <- Diag(e^{G_n}) S^T + (E o e^{G_n - G})^T X
#pragma unroll
        for (int t = 0; t < NCT; ++t) {
            st[t] = st[t] * *reinterpret_cast<const f32x4 *>(sEG + 16 * t + 4 * lq);
            tok_prod(sU, D * LC, xh, xl, st[t], t);
        }
        __syncthreads();
        // ---- phase 5: S^T <- S^T + (K o e^{G_n - G})^T Z
#pragma unroll
        for (int t = 0; t < NCT; ++t) tok_prod(sW, D * LC, zh, zl, st[t], t);
        __syncthreads();
    }
    if (S_T) {
#pragma unroll
        for (int t = 0; t < NCT; ++t)
            *reinterpret_cast<f32x4 *>(S_T + ((size_t)uh * D + vcol) * D + 16 * t + 4 * lq) = st[t];
    }
}

template <int D, typename TI, typename TO>
hipError_t launch_gdn2_t(int units, int T, int H, const int32_t *cu, const void *q,
                         const void *k, const void *v, const float *la, const float *erase,
                         const float *write, const float *S0, void *o, float *S_T, bf16 *ws,
                         long nslots, hipStream_t st) {
    const int varlen = cu != nullptr;
    const int NC = varlen ? 0 : (T + BC - 1) / BC;
    const size_t nch = (size_t)nslots * H;
    if (nch > 0)
        hipLaunchKernelGGL((gdn2_prep_kernel<D, TI>), dim3((unsigned)std::min<size_t>(nch, 256)),
                           dim3(512), 0, st, T, H, units, NC, varlen, cu, (const TI *)q,
                           (const TI *)k, la, erase, ws, (int)nch);
    const long nuh = (long)units * H;
    const int xcd_map = nuh % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((gdn2_fwd_kernel<D, TI, TO>), dim3((unsigned)(nuh * (D / 64))), dim3(512),
                       0, st, T, H, NC, varlen, xcd_map, cu, (const TI *)v, write, S0, ws,
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
    return sizeof(bf16) * (size_t)nslots * H * per;
}

hipError_t launch_gdn2_fwd(int units, int T, int H, int d, bool io_bf16, bool o_bf16,
                           const int32_t *cu, const void *q, const void *k, const void *v,
                           const float *la, const float *erase, const float *write,
                           const float *S0, void *o, float *S_T, void *ws, hipStream_t st) {
    const long nslots = cu ? (long)T / BC + units + 1 : (long)units * ((T + BC - 1) / BC);
    bf16 *w = (bf16 *)ws;
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
