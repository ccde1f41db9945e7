// Chunkwise forward of the gated delta rule on gfx950 matrix cores (bf16
// inputs, fp32 state and accumulation).
//
// Method: the extended WY/UT chunk algorithm ("Gated Delta Networks:
// Improving Mamba2 with Delta Rule", research-map summary, section
// "Approach"; blog "Gated DeltaNet: Harmonizing Gating and the Delta Rule for
// Superior Linear RNNs", section "Hardware-Efficient Training").  For one
// chunk of C = 64 tokens (zero-padded at a ragged end) and the state S
// (d_v x d_k) that enters it, with g the chunk-local prefix sum of log alpha:
//   (1) g_r = sum_{s<=r} log alpha_s
//   (2) A[r,i] = beta_r e^{g_r-g_i} (k_r . k_i) for i < r;  T = (I + A)^{-1}
//   (3) U = T diag(beta) V,  W = T diag(beta e^g) K
//   (4) Delta = U - W S^T;   S <- e^{g_C} S + Delta^T diag(e^{g_C-g}) K
//   (5) O = diag(e^g) Q S^T + (tril(Q K^T) o e^{g_r-g_i}) Delta
// Neither U nor W is formed: U - W S^T = T diag(beta) (V - diag(e^g) K S^T),
// so the kernel keeps the one factor T_U = T diag(beta) and multiplies it
// into Z = V - diag(e^g) Y with Y = K S^T.
//
// Work split.  One workgroup of 8 waves owns one (sequence, head, 64-column
// slice of d_v) and walks its chunks in order, so q, k, v and the gates are
// read once and o is written once.  Waves 0-3 ("producers") prepare chunk
// n+1 -- global prefetch, gate prefix, K K^T and Q K^T on MFMA, the 64x64
// unit-lower inverse (four 16x16 diagonal blocks by blocked forward
// substitution in fp32, one per wave, then the off-diagonal blocks
// T_ij = -T_ii sum_k A_ik T_kj on 16x16 MFMA, one block column per wave), the
// factor T diag(beta) as a bf16 hi + lo pair and K^T -- while waves
// 4-7 ("consumers") run the state chain of chunk n.  Consumer c owns 16
// columns of the slice and keeps its S^T columns (d_k x 16, fp32) in MFMA
// accumulators; S^T, Y and Delta feed the next MFMA straight from registers
// (layouts in gdn_common.h).  An iteration has three barrier-separated
// phases; every LDS buffer is written by one phase and read in later ones
// before it is overwritten (K^T and the gates are double-buffered):
//   phase  producers (chunk n+1)               consumers (chunk n)
//   1      store q,k; each wave forms K^T of   Delta = T diag(beta) Z, Delta~
//          its own 16 tokens; prefetch q,k
//   2      store v, prefetch v; K K^T -> A;    S <- e^{g_C} S + K^T Delta~,
//          each wave inverts and converts      P Delta, write o
//          the diagonal block of A it formed
//   3      off-diagonal T and its conversion,  Q S^T, Y = K S^T and
//          Q K^T -> P, gate prefix of n+2      Z = V - diag(e^g) Y, chunk n+1
// Global loads and stores go through buffer resources sized to the valid
// rows of the chunk: rows past a ragged end read as zero and their stores
// are dropped by the hardware range check, so no lane branches on bounds.
// Precision: outputs are heavy-tailed (max |o| is 10-20x its RMS), so the
// operands carrying the state or the corrected values are split into
// hi + lo bf16 pairs (S^T, Z, Delta, Delta~, P, and A, T and T diag(beta)
// in the UT transform) and o is written in fp32
// (or bf16 on request).
#include "gdn_common.h"

namespace gdn {

template <int N> struct IntC { static constexpr int value = N; };

constexpr int kC = 64;     // chunk length
constexpr int kDVT = 64;   // d_v columns per workgroup (16 per consumer wave)
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ float exp_neg(float x) {   // e^x for x <= 0
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Gate prologue on the hardware transcendentals (v_exp_f32, v_log_f32,
// v_rcp_f32, each within a few ulp).  -softplus(a) = -(max(a, 0) + log1p(y))
// with y = e^{-|a|} in (0, 1]; log1p(y) = ln(t) y / (t - 1) with t = 1 + y
// undoes the rounding of t (and is y itself once t rounds to 1).
__device__ __forceinline__ float neg_softplus_hw(float a) {
    const float y = exp_neg(-fabsf(a));
    const float t = 1.f + y;
    const float l1p = t == 1.f ? y
                               : __builtin_amdgcn_logf(t) * 0.6931471805599453f * y *
                                     __builtin_amdgcn_rcpf(t - 1.f);
    return -(fmaxf(a, 0.f) + l1p);
}
__device__ __forceinline__ float sigmoid_hw(float b) {   // 1 / (1 + e^{-b}); 0 as b -> -inf
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-b * 1.4426950408889634f));
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
    return bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return to_bf16x4(x[0], x[1], x[2], x[3]); }

// hi + lo splits (x = hi + lo + below 2^-16 |x|, hi = bf16(x) rounded to
// nearest even, lo = bf16(x - hi)) with the residual x - hi taken by one
// v_dot2_f32_bf16 per element: hi_pair . (-1, 0) + a and hi_pair . (0, -1) + b
// are exact (the products are exact and x - hi is representable), in place
// of rebuilding hi as fp32 and subtracting.  The two selector pairs live in
// registers: as an inline constant the compiler encodes (-1, 0) as the fp32
// -1.0, which the hardware reads as the pair (0, -1).
struct SplitSel {
    uint32_t lo, hi;   // bf16 pairs (-1, 0) and (0, -1)
};
__device__ __forceinline__ SplitSel split_sel() {
    SplitSel m;
    asm("v_mov_b32 %0, 0xbf80" : "=v"(m.lo));
    asm("v_mov_b32 %0, 0xbf800000" : "=v"(m.hi));
    return m;
}
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_pair2(float a, float b, const SplitSel &m, uint32_t &hi,
                                            uint32_t &lo) {
    const bf16x2 h = bf16x2{(bf16)a, (bf16)b};
    hi = __builtin_bit_cast(uint32_t, h);
    const float ra = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m.lo), a, false);
    const float rb = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m.hi), b, false);
    lo = __builtin_bit_cast(uint32_t, bf16x2{(bf16)ra, (bf16)rb});
}
__device__ __forceinline__ void split4(f32x4 x, const SplitSel &m, bf16x4 &hi, bf16x4 &lo) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    uint32_t h0, h1, l0, l1;
    split_pair2(x[0], x[1], m, h0, l0);
    split_pair2(x[2], x[3], m, h1, l1);
    hi = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
    lo = __builtin_bit_cast(bf16x4, u32x2{l0, l1});
}
// Two D tiles (rows 0-15 and 16-31 of a 32-row block) as a D-order operand pair.
__device__ __forceinline__ void split8(f32x4 d0, f32x4 d1, const SplitSel &m, bf16x8 &hi,
                                       bf16x8 &lo) {
    bf16x4 h0, l0, h1, l1;
    split4(d0, m, h0, l0);
    split4(d1, m, h1, l1);
    hi = cat(h0, h1);
    lo = cat(l0, l1);
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// Operand tiles in LDS ("D-order rows").  An MFMA operand fragment takes, per
// lane group lg, the k values 4lg..4lg+3 and 16+4lg..16+4lg+3 of a 32-wide
// k block (the order in which D-layout results feed the next product).  Row
// tiles store each 32-column block with its 4-column chunks in the order
// 0,4,1,5,2,6,3,7, so such a fragment is one 16-byte read.
__device__ __forceinline__ int dcol(int c) {   // D-order position of column c
    return (c & ~31) | (((c >> 2) & 3) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}
// Rows are unpadded, W elements long, with their 16-byte chunks XOR-permuted
// by row: 16 consecutive rows then put a 16-byte chunk (fragment reads) or
// an 8-byte piece (stores of D-layout results, 16 rows x 8 bytes) on
// distinct banks.  (Padded rows measured 1.2-1.3x slower for the reads and
// about 2x slower for the 8-byte stores.)
template <int W> __device__ __forceinline__ int tswz(int r) {
    return W == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int W> __device__ __forceinline__ int tposd(int r, int d) {   // D-order position d
    return r * W + 8 * ((d >> 3) ^ tswz<W>(r)) + (d & 7);
}
template <int W> __device__ __forceinline__ int tpos(int r, int c) {    // natural column c
    return tposd<W>(r, dcol(c));
}
// Operand fragment of a D-order row tile of width W: rows row0..row0+15
// (row0 a multiple of 16), k block ks.
template <int W>
__device__ __forceinline__ bf16x8 tfrag(const bf16 *x, int row0, int ks, int lane) {
    return *reinterpret_cast<const bf16x8 *>(x + tposd<W>(row0 + (lane & 15), 32 * ks + 8 * (lane >> 4)));
}
// The V slice, read only as a column gather, sits unpadded with its 8-byte
// chunks permuted within each row: chunk c of row r is stored at chunk
// c ^ swz(r), which keeps the transpose reads (4 consecutive rows x 4
// consecutive chunks per 16 lanes) on distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}
__device__ __forceinline__ bf16x8 buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store(float x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(bf16 x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, off, 0, 0);
}

// Input prologue, PRO bit 0 (NQK): q and k arrive unnormalised and the
// kernel L2-normalises them per token; bit 1 (GATES): log_alpha and beta hold
// the pre-activations a and b, and the kernel uses log alpha = -softplus(a),
// beta = sigmoid(b).
template <int DK, typename TO, int PRO>
__global__ __launch_bounds__(512, 1) void chunk_mfma_kernel(
    int T, int H, int DV, int varlen, int xcd_map,
    const int32_t *__restrict__ cu_seqlens,
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const float *__restrict__ log_alpha, const float *__restrict__ beta,
    const float *__restrict__ S0, TO *__restrict__ o, float *__restrict__ S_T) {
    constexpr int C = kC;
    constexpr bool NQK = (PRO & 1) != 0, GATES = (PRO & 2) != 0;
    constexpr int NKS = DK / 32;        // 32-wide k-steps over d_k
    constexpr int NMT = DK / 16;        // 16-row tiles over d_k
    // Row length (elements) of A, whose 16x16x16 operands are 8-byte reads of
    // 16 rows (2 mod 4 dwords puts those on distinct bank pairs).
    constexpr int LDC = C + 4;
    constexpr int BLK = 260;            // stride of the 16x16 fp32 diagonal blocks (4 banks apart)
    constexpr int QK_PIECES = C * DK / 8;            // 16-byte pieces of a q or k chunk
    constexpr int QK_PER_THR = QK_PIECES / 256;
    constexpr int QK_PPR = DK / 8;                   // 16-byte pieces per row
    static_assert(QK_PER_THR * (64 / QK_PPR) == 16, "a producer wave owns 16 rows of q and k");
    constexpr int V_PER_THR = C * kDVT / 8 / 256;
    static_assert(QK_PIECES % 256 == 0 && V_PER_THR * 256 == C * kDVT / 8, "piece split");

    __shared__ __attribute__((aligned(16))) bf16 sQ[C * DK];        // Q, D-order rows
    __shared__ __attribute__((aligned(16))) bf16 sK[C * DK];        // K, D-order rows
    __shared__ __attribute__((aligned(16))) bf16 sKT[2][DK * C];    // K^T, chunks m and m-1
    __shared__ __attribute__((aligned(16))) bf16 sV[C * kDVT];      // V slice (swizzled)
    __shared__ __attribute__((aligned(16))) bf16 sA[C * LDC];       // A, off-diagonal blocks, hi
    __shared__ __attribute__((aligned(16))) bf16 sAl[C * LDC];      //   and lo parts
    __shared__ __attribute__((aligned(16))) float sAd[4 * BLK];     // A diag blocks, [b][col][row]
    __shared__ __attribute__((aligned(16))) float sTd[4 * BLK];     // T diag blocks, [b][row][col]
    __shared__ __attribute__((aligned(16))) float sTdT[4 * BLK];    // T diag blocks, [b][col][row]
    // the C x C factors, D-order rows
    // as hi + lo pairs
    __shared__ __attribute__((aligned(16))) bf16 sTU[C * C];        // T diag(beta), hi
    __shared__ __attribute__((aligned(16))) bf16 sTUl[C * C];       //   lo
    // P = tril(QK^T) o decay as hi + lo, chunks m and m-1
    __shared__ __attribute__((aligned(16))) bf16 sPh[C * C];
    __shared__ __attribute__((aligned(16))) bf16 sPl[C * C];
    // per-token values of a chunk, double-buffered: g, e^g, beta,
    // e^{g_C - g}, and (prologue) 1/|q|, 1/|k|
    __shared__ __attribute__((aligned(16))) float sG[2][6][C];

    // Workgroup -> (unit, head, d_v slice).  With xcd_map the slices of one
    // (unit, head) land on the same XCD (workgroups are dealt to the 8 XCDs
    // round-robin), so the repeated reads of q and k hit that XCD's L2.
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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int lm = lane & 15, lg = lane >> 4;
    const SplitSel sm = split_sel();

    // Operand element (i, k) = V[32 ks + k][16 cb + i] (k in D-order) of the
    // swizzled V slice: a column gather by two transpose reads.
    auto v_frag = [&](int cb, int ks) {
        const int j = lm >> 2, q4 = lm & 3;
        const bf16 *p = sV + (32 * ks + 4 * lg + j) * kDVT + 4 * ((4 * cb + q4) ^ ((j << 2) | lg));
        return cat(lds_read_tr(p), lds_read_tr(p + 16 * kDVT));
    };
    // 16x16x16 operand holding the identity: D = X I turns X (given as an A
    // operand: lane (lm, lg) holds row lm, columns 4lg..4lg+3) into D layout
    // (lane holds rows 4lg..4lg+3 of column lm), i.e. transposes lane data.
    bf16x4 eye;
#pragma unroll
    for (int s = 0; s < 4; ++s) eye[s] = (bf16)((4 * lg + s == lm) ? 1.f : 0.f);

    long row0, L;
    if (varlen) {
        row0 = cu_seqlens[unit];
        L = (long)cu_seqlens[unit + 1] - row0;
    } else {
        row0 = (long)unit * T;
        L = T;
    }
    const int N = (int)((L + C - 1) / C);
    // first token (absolute row) and valid rows of chunk c
    auto crow = [&](int c) -> size_t { return (size_t)(row0 + (long)c * C); };
    // (0 past the last chunk: prefetches there read nothing and return zeros)
    auto cvalid = [&](int c) -> uint32_t {
        return (uint32_t)max(0L, min((long)C, L - (long)c * C));
    };

    // Upper off-diagonal blocks of the LDS factors are never written: zero them once.
    for (int e = tid; e < C * C / 2; e += 512) {
        reinterpret_cast<uint32_t *>(sTU)[e] = 0u;
        reinterpret_cast<uint32_t *>(sTUl)[e] = 0u;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if (b == 0) {
                reinterpret_cast<uint32_t *>(sPh)[e] = 0u;
                reinterpret_cast<uint32_t *>(sPl)[e] = 0u;
            }
        }
    }
    __syncthreads();

    // Producers and consumers run separate loops (so each role's registers
    // are allocated on their own); both pass the same four barriers per
    // iteration, N + 1 times.
    if (wave < 4) {
        const int pw = wave;       // producer wave 0..3
        const int ptid = tid;      // producer thread 0..255
        bf16x8 pq[QK_PER_THR], pk[QK_PER_THR], pv[V_PER_THR];
        float pla = 0.f, pbe = 0.f;
        bool pvalid = false;   // this lane's token exists (gate pre-activations)
        // The next chunk's loads are issued on every iteration, also past the
        // last chunk (zero valid rows: the range check turns them into zeros
        // without a memory access), so the compiler's wait counts can rely on
        // them: a conditional load makes it wait for every outstanding load
        // before the stores of the current chunk.
        auto prefetch_qk = [&](int c) {
            const uint32_t nv = cvalid(c);
            const size_t t0 = nv ? crow(c) : crow(0);
            const rsrc_t rq = make_rsrc(q + (t0 * H + h) * DK, nv * H * DK * 2);
            const rsrc_t rk = make_rsrc(k + (t0 * H + h) * DK, nv * H * DK * 2);
#pragma unroll
            for (int i = 0; i < QK_PER_THR; ++i) {
                const int r = 16 * pw + i * (64 / QK_PPR) + lane / QK_PPR, p = lane % QK_PPR;
                const uint32_t off = (uint32_t)(r * H * DK + 8 * p) * 2;
                pq[i] = buf_load16(rq, off);
                pk[i] = buf_load16(rk, off);
            }
            if (pw == 3) {
                const rsrc_t ra = make_rsrc(log_alpha + t0 * H + h, nv * H * 4);
                const rsrc_t rb = make_rsrc(beta + t0 * H + h, nv * H * 4);
                pla = buf_load4(ra, (uint32_t)(lane * H) * 4);
                pbe = buf_load4(rb, (uint32_t)(lane * H) * 4);
                pvalid = (uint32_t)lane < nv;
            }
        };
        // Gate prefix of the prefetched chunk into gate buffer `buf`, one token
        // per lane of wave 3 (padded tokens add 0).
        auto scan_gates = [&](int buf) {
            float x = pla, b = pbe;
            if constexpr (GATES) {   // padded tokens keep log alpha = beta = 0
                x = pvalid ? neg_softplus_hw(x) : 0.f;
                b = pvalid ? sigmoid_hw(b) : 0.f;
            }
            x = wave_scan64(x);
            const float gC = lane63(x);
            sG[buf][0][lane] = x;
            sG[buf][1][lane] = exp_neg(x);
            sG[buf][2][lane] = b;
            sG[buf][3][lane] = exp_neg(gC - x);
        };
        auto prefetch_v = [&](int c) {
            const uint32_t nv = cvalid(c);
            const size_t t0 = nv ? crow(c) : crow(0);
            const rsrc_t rv = make_rsrc(v + (t0 * H + h) * DV + dv0, nv * H * DV * 2);
#pragma unroll
            for (int i = 0; i < V_PER_THR; ++i) {
                const int e = ptid + 256 * i, r = e / (kDVT / 8), p = e % (kDVT / 8);
                pv[i] = buf_load16(rv, (uint32_t)(r * H * DV + 8 * p) * 2);
            }
        };
        if (N > 0) {
            prefetch_qk(0);
            prefetch_v(0);
            if (pw == 3) scan_gates(0);   // later chunks are scanned a phase ahead
        }
        // Iterations n = -1 .. N-2 prepare chunk m = n + 1; the last one
        // (n = N - 1, nothing left to prepare) only passes the barriers, after
        // the loop, so that every load and store inside the loop is
        // unconditional and the compiler's wait counts stay exact.
        for (int n = -1; n < N - 1; ++n) {
            const int m = n + 1;           // chunk being prepared
            constexpr bool prep = true;
            const int gb = m & 1;          // gate buffer of chunk m
            // ================================ phase 1
            if (prep) {
#pragma unroll
                for (int i = 0; i < QK_PER_THR; ++i) {
                    const int r = 16 * pw + i * (64 / QK_PPR) + lane / QK_PPR, p = lane % QK_PPR;
                    const int c0 = tpos<DK>(r, 8 * p), c1 = tpos<DK>(r, 8 * p + 4);
                    *reinterpret_cast<bf16x4 *>(sQ + c0) = bf16x4{pq[i][0], pq[i][1], pq[i][2], pq[i][3]};
                    *reinterpret_cast<bf16x4 *>(sQ + c1) = bf16x4{pq[i][4], pq[i][5], pq[i][6], pq[i][7]};
                    *reinterpret_cast<bf16x4 *>(sK + c0) = bf16x4{pk[i][0], pk[i][1], pk[i][2], pk[i][3]};
                    *reinterpret_cast<bf16x4 *>(sK + c1) = bf16x4{pk[i][4], pk[i][5], pk[i][6], pk[i][7]};
                }
                prefetch_qk(m + 1);
                // K^T of this wave's 16 tokens (the rows it has just stored), all
                // of d_k, by identity products on 16x16 blocks, into the buffer
                // of chunk m (the consumers read chunk n's in phase 2).
                {
                    bf16x4 kb[DK / 16];
#pragma unroll
                    for (int cb = 0; cb < DK / 16; ++cb)
                        kb[cb] = *reinterpret_cast<const bf16x4 *>(sK + tpos<DK>(16 * pw + lm, 16 * cb + 4 * lg));
                    f32x4 kt[DK / 16];
#pragma unroll
                    for (int cb = 0; cb < DK / 16; ++cb) kt[cb] = mfma16(kb[cb], eye, zero4());
#pragma unroll
                    for (int cb = 0; cb < DK / 16; ++cb)
                        *reinterpret_cast<bf16x4 *>(sKT[m & 1] + tpos<C>(16 * cb + lm, 16 * pw + 4 * lg)) =
                            to_bf16x4(kt[cb]);
                }
                if constexpr (NQK) {
                    // |q_r|^2 and |k_r|^2 of this wave's 16 rows: the diagonal of
                    // Q_b Q_b^T and K_b K_b^T (one fragment serves as both
                    // operands).  Row lm's entry sits in lane (lm, lm >> 2),
                    // register lm & 3.
                    f32x4 nq = zero4(), nk = zero4();
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const bf16x8 fq = tfrag<DK>(sQ, 16 * pw, ks, lane);
                        const bf16x8 fk = tfrag<DK>(sK, 16 * pw, ks, lane);
                        nq = mfma32(fq, fq, nq);
                        nk = mfma32(fk, fk, nk);
                    }
                    if ((lm >> 2) == lg) {
                        const int j = lm & 3;
                        const float sq = j == 0 ? nq[0] : j == 1 ? nq[1] : j == 2 ? nq[2] : nq[3];
                        const float sk = j == 0 ? nk[0] : j == 1 ? nk[1] : j == 2 ? nk[2] : nk[3];
                        sG[m & 1][4][16 * pw + lm] = __builtin_amdgcn_rsqf(fmaxf(sq, 1e-12f));
                        sG[m & 1][5][16 * pw + lm] = __builtin_amdgcn_rsqf(fmaxf(sk, 1e-12f));
                    }
                }
            }
            __syncthreads();
            // Diagonal block b of T diag(beta), one (row, 4 columns) per lane.
            auto diag_conv = [&](int b) {
                const int r = lane >> 2, c4 = 4 * (lane & 3);
                const f32x4 tv = ld4(sTd + b * BLK + r * 16 + c4);
                const f32x4 bc = ld4(&sG[gb][2][16 * b + c4]);
                f32x4 tu;
#pragma unroll
                for (int s = 0; s < 4; ++s) tu[s] = (c4 + s <= r) ? tv[s] * bc[s] : 0.f;
                bf16x4 uh, ul;
                split4(tu, sm, uh, ul);
                const int off = tpos<C>(16 * b + r, 16 * b + c4);
                *reinterpret_cast<bf16x4 *>(sTU + off) = uh;
                *reinterpret_cast<bf16x4 *>(sTUl + off) = ul;
            };
            // K K^T and Q K^T tiles (ti, tj), tj <= ti, 10 of each: the K K^T
            // part (A) in phase 2, the Q K^T part (P) in phase 3 (the consumers
            // read P of chunk m in phase 2 of the next iteration); a wave loads
            // each 16-row block of K or Q it needs once.
            typedef bf16x8 Frag[NKS];
            auto load_q = [&](int blk, Frag &f) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) f[ks] = tfrag<DK>(sQ, 16 * blk, ks, lane);
            };
            auto load_k = [&](int blk, Frag &f) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) f[ks] = tfrag<DK>(sK, 16 * blk, ks, lane);
            };
            // A tile forms both its K K^T part (A) and its Q K^T part (P), or
            // one of them (DO: 1 = A only, 2 = P only, 3 = both).
            const IntC<1> A_ONLY;
            const IntC<2> P_ONLY;
            auto tile = [&](const int ti, const int tj, const Frag &fKj, const Frag &fKi,
                            const Frag &fQi, auto doc) {
                constexpr int DO = decltype(doc)::value;
                constexpr bool doA = (DO & 1) != 0, doP = (DO & 2) != 0;
                f32x4 G = zero4(), PT = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if constexpr (doA) G = mfma32(fKj[ks], fKi[ks], G);    // k_i . k_r,  i = 16 tj + 4 lg + j, r = 16 ti + lm
                    if constexpr (doP) PT = mfma32(fKj[ks], fQi[ks], PT);  // k_i . q_r
                }
                const int r = 16 * ti + lm, i0 = 16 * tj + 4 * lg;
                const float gr = sG[gb][0][r], br = sG[gb][2][r];
                const f32x4 gi = ld4(&sG[gb][0][i0]);
                if constexpr (NQK) {   // normalised rows: scale the Gram entries
                    const f32x4 iki = ld4(&sG[gb][5][i0]);
                    G = G * (sG[gb][5][r] * iki);
                    PT = PT * (sG[gb][4][r] * iki);
                }
                f32x4 dec;   // e^{g_r - g_i} on and below the diagonal, else 0
#pragma unroll
                for (int j = 0; j < 4; ++j) dec[j] = (i0 + j <= r) ? exp_neg(gr - gi[j]) : 0.f;
                if constexpr (doP) {
                    bf16x4 ph, pl;
                    split4(dec * PT, sm, ph, pl);
                    *reinterpret_cast<bf16x4 *>(sPh + tpos<C>(r, i0)) = ph;
                    *reinterpret_cast<bf16x4 *>(sPl + tpos<C>(r, i0)) = pl;
                }
                if (!doA) {
                } else if (ti > tj) {
                    bf16x4 ah, al;
                    split4(br * dec * G, sm, ah, al);
                    *reinterpret_cast<bf16x4 *>(sA + r * LDC + i0) = ah;
                    *reinterpret_cast<bf16x4 *>(sAl + r * LDC + i0) = al;
                } else {
                    // Diagonal tile: K K^T is symmetric, so the registers also
                    // hold rows rr = i0 + j of column r; store A's block
                    // transposed (column contiguous) for the substitution.
                    const f32x4 brr = ld4(&sG[gb][2][i0]);
                    f32x4 d4;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        d4[j] = (i0 + j > r) ? brr[j] * exp_neg(gi[j] - gr) * G[j] : 0.f;
                    *reinterpret_cast<f32x4 *>(sAd + ti * BLK + lm * 16 + 4 * lg) = d4;
                }
            };
            // ================================ phase 2
            if (prep) {
                // V slice of chunk m (the consumers read chunk n's in phase 1),
                // then the next chunk's loads
#pragma unroll
                for (int i = 0; i < V_PER_THR; ++i) {
                    const int e = ptid + 256 * i, r = e / (kDVT / 8), p = e % (kDVT / 8);
                    bf16 *dv = sV + r * kDVT;
                    const int f = swz(r);
                    *reinterpret_cast<bf16x4 *>(dv + 4 * ((2 * p) ^ f)) = bf16x4{pv[i][0], pv[i][1], pv[i][2], pv[i][3]};
                    *reinterpret_cast<bf16x4 *>(dv + 4 * ((2 * p + 1) ^ f)) = bf16x4{pv[i][4], pv[i][5], pv[i][6], pv[i][7]};
                }
                prefetch_v(m + 1);
                // The ten A blocks: each wave its diagonal block first (its
                // inverse follows), and one or two below the diagonal.
                if (pw == 0) {
                    Frag k0, k1, k3;
                    load_k(0, k0); load_k(1, k1); load_k(3, k3);
                    tile(0, 0, k0, k0, k0, A_ONLY);
                    tile(1, 0, k0, k1, k1, A_ONLY);
                    tile(3, 0, k0, k3, k3, A_ONLY);
                } else if (pw == 1) {
                    Frag k1, k2, k3;
                    load_k(1, k1); load_k(2, k2); load_k(3, k3);
                    tile(1, 1, k1, k1, k1, A_ONLY);
                    tile(2, 1, k1, k2, k2, A_ONLY);
                    tile(3, 2, k2, k3, k3, A_ONLY);
                } else if (pw == 2) {
                    Frag k0, k2;
                    load_k(2, k2); load_k(0, k0);
                    tile(2, 2, k2, k2, k2, A_ONLY);
                    tile(2, 0, k0, k2, k2, A_ONLY);
                } else {
                    Frag k1, k3;
                    load_k(3, k3); load_k(1, k1);
                    tile(3, 3, k3, k3, k3, A_ONLY);
                    tile(3, 1, k1, k3, k3, A_ONLY);
                }
                // Diagonal blocks: this wave computed tile (pw, pw) of A above and
                // inverts and converts that block itself (no barrier needed).
                {
                    // Diagonal block b = pw of T = (I + A)^{-1} in fp32.  Lane
                    // (column cl, row group g) holds rows 4g..4g+3 of column cl;
                    // blocked forward substitution over the four row groups, with
                    // each solved group broadcast within its lane quad by DPP.
                    // The block's columns of A are contiguous in sAd.
                    const int b = pw, cl = lane >> 2, g = lane & 3;
                    const float *Ad = sAd + b * BLK;
                    f32x4 x;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) x[rr] = (4 * g + rr == cl) ? 1.f : 0.f;
                    // all loads first: acol[s][k][rr] = A[4 g + rr][4 s + k] of the block
                    f32x4 acol[4][4];
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) acol[sb][kk] = ld4(Ad + (4 * sb + kk) * 16 + 4 * g);
                    auto group = [&](auto sbc) {
                        constexpr int sb = decltype(sbc)::value;
                        const f32x4 *col = acol[sb];
                        // rows of group sb: solve the 4x4 diagonal sub-block
                        f32x4 t = x;
#pragma unroll
                        for (int c = 0; c < 3; ++c)
#pragma unroll
                            for (int rr = c + 1; rr < 4; ++rr) t[rr] -= col[c][rr] * t[c];
                        const bool mine = g == sb, later = g > sb;   // lane-varying: selects, not branches
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) x[rr] = mine ? t[rr] : x[rr];
                        if constexpr (sb < 3) {
                            f32x4 xb;   // the solved rows 4 sb..4 sb+3 of this column
#pragma unroll
                            for (int kk = 0; kk < 4; ++kk)
                                xb[kk] = __int_as_float(__builtin_amdgcn_mov_dpp(
                                    __float_as_int(x[kk]), sb * 0x55, 0xf, 0xf, false));
                            // later groups subtract their rows' share of it
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) {
                                const float y = x[rr] - ((col[0][rr] * xb[0] + col[1][rr] * xb[1]) +
                                                         (col[2][rr] * xb[2] + col[3][rr] * xb[3]));
                                x[rr] = later ? y : x[rr];
                            }
                        }
                    };
                    group(IntC<0>{});
                    group(IntC<1>{});
                    group(IntC<2>{});
                    group(IntC<3>{});
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) sTd[b * BLK + (4 * g + rr) * 16 + cl] = x[rr];
                    *reinterpret_cast<f32x4 *>(sTdT + b * BLK + cl * 16 + 4 * g) = x;
                }
                diag_conv(pw);
            }
            __syncthreads();
            // ================================ phase 3
            // Off-diagonal blocks of block column j, top to bottom:
            // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj (16x16x16 MFMA).  Column j
            // only needs its own blocks and the diagonal ones, so producer wave
            // j < 3 computes column j with no exchange between waves.
            // Every factor is carried as a hi + lo pair and each product as the
            // three piece products hi*hi + lo*hi + hi*lo: with keys repeated or
            // nearly collinear inside a chunk the entries of A approach beta
            // and T's products cancel, so single bf16 roundings of A, T or the
            // factors cost several per cent of o.
            auto column = [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                bf16x4 Bh[4], Bl[4];   // B operands: T_jj, then T_kj (k > j), hi + lo
                f32x4 RT[4];           // RT[k] = T_kj in D layout, k > j
                bf16x4 Ah[4][4], Al[4][4], Th[4], Tl[4];   // A_ik and T_ii (i > j), hi + lo
                split4(ld4(sTdT + j * BLK + lm * 16 + 4 * lg), sm, Bh[j], Bl[j]);
#pragma unroll
                for (int i = j + 1; i < 4; ++i) {
#pragma unroll
                    for (int kk = j; kk < i; ++kk) {
                        const int aoff = (16 * i + lm) * LDC + 16 * kk + 4 * lg;
                        Ah[i][kk] = *reinterpret_cast<const bf16x4 *>(sA + aoff);
                        Al[i][kk] = *reinterpret_cast<const bf16x4 *>(sAl + aoff);
                    }
                    split4(ld4(sTd + i * BLK + lm * 16 + 4 * lg), sm, Th[i], Tl[i]);
                }
                // Y_i = sum_k A_ik T_kj, kept as two accumulators per block (the
                // hi*hi + lo*hi and the hi*lo pieces): the T_jj terms of every
                // block start at once, and each solved block T_kj is added to
                // all later blocks before the next one is solved, so only one
                // product per block sits on the column's dependency chain.
                f32x4 Ya[4], Yc[4];
#pragma unroll
                for (int i = j + 1; i < 4; ++i) {
                    Ya[i] = mfma16(Ah[i][j], Bh[j], zero4());
                    Yc[i] = mfma16(Ah[i][j], Bl[j], zero4());
                    Ya[i] = mfma16(Al[i][j], Bh[j], Ya[i]);
                }
#pragma unroll
                for (int k = j + 1; k < 4; ++k) {
                    bf16x4 ybh, ybl;
                    split4(Ya[k] + Yc[k], sm, ybh, ybl);
                    f32x4 r = mfma16(Th[k], ybh, zero4());
                    const f32x4 r2 = mfma16(Th[k], ybl, zero4());
                    r = mfma16(Tl[k], ybh, r);
                    RT[k] = -(r + r2);
                    split4(RT[k], sm, Bh[k], Bl[k]);
#pragma unroll
                    for (int i = k + 1; i < 4; ++i) {
                        Ya[i] = mfma16(Ah[i][k], Bh[k], Ya[i]);
                        Yc[i] = mfma16(Ah[i][k], Bl[k], Yc[i]);
                        Ya[i] = mfma16(Al[i][k], Bh[k], Ya[i]);
                    }
                }
                // Scale column c = 16 j + lm by beta_c, split into a hi + lo pair,
                // and transpose with identity products (exact) so that each lane
                // writes 4 consecutive columns of one row.
                const float bc = sG[gb][2][16 * j + lm];
#pragma unroll
                for (int i = j + 1; i < 4; ++i) {
                    bf16x4 uh, ul;
                    split4(RT[i] * bc, sm, uh, ul);
                    const int off = tpos<C>(16 * i + lm, 16 * j + 4 * lg);
                    *reinterpret_cast<bf16x4 *>(sTU + off) = to_bf16x4(mfma16(uh, eye, zero4()));
                    *reinterpret_cast<bf16x4 *>(sTUl + off) = to_bf16x4(mfma16(ul, eye, zero4()));
                }
            };
            if (prep) {
                // T's block column j on wave j < 3 (column 0 is the longest), the
                // ten P blocks on the other waves (none on wave 0, two on wave
                // 1, four on waves 2 and 3), and chunk m+1's gate prefix on
                // wave 3, into the buffer chunk n used (the consumers are done
                // with it; past the last chunk it is unused)
                if (pw == 0) {
                    column(IntC<0>{});
                } else if (pw == 1) {
                    column(IntC<1>{});
                    Frag k0, k1, q1;
                    load_k(0, k0); load_k(1, k1); load_q(1, q1);
                    tile(1, 0, k0, k1, q1, P_ONLY);
                    tile(1, 1, k1, k1, q1, P_ONLY);
                } else if (pw == 2) {
                    column(IntC<2>{});
                    Frag k0, k1, k2, q0, q2;
                    load_k(0, k0); load_q(0, q0);
                    tile(0, 0, k0, k0, q0, P_ONLY);
                    load_k(1, k1); load_k(2, k2); load_q(2, q2);
                    tile(2, 0, k0, k2, q2, P_ONLY);
                    tile(2, 1, k1, k2, q2, P_ONLY);
                    tile(2, 2, k2, k2, q2, P_ONLY);
                } else {
                    scan_gates(gb ^ 1);
                    Frag kj, q3;
                    load_q(3, q3);
#pragma unroll
                    for (int tj = 0; tj < 4; ++tj) {
                        load_k(tj, kj);
                        tile(3, tj, kj, kj, q3, P_ONLY);
                    }
                }
            }
            __syncthreads();
        }
        if (N > 0) {   // iteration n = N - 1: the consumers finish the last chunk
            __syncthreads();
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    // ---------------------------------------------------------------- consumers
    const int cw = 16 * (wave - 4);     // first column of this wave within the slice
    const int dvw = dv0 + cw + lm;      // this lane's d_v column
    const size_t sbase = ((size_t)unit * H + h) * DV * DK;
    f32x4 st[NMT];      // st[mt][j] = S^T[16 mt + 4 lg + j][dvw]
    f32x4 QS[4];        // diag(e^g) Q S^T of the next chunk, rows 16 mr + 4 lg + j
    bf16x8 zh[2], zl[2];  // Z = V - diag(e^g) K S^T of the next chunk, hi + lo (D order)
    bf16x8 th[2], tl[2];  // Delta~ = diag(e^{g_C - g}) Delta, hi + lo (D order)
    bf16x8 dh[2], dl[2];  // Delta, hi + lo
    bf16x8 sh[NKS], sl[NKS];  // S^T, hi + lo
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        st[mt] = zero4();
        if (S0) st[mt] = ld4(S0 + sbase + (size_t)dvw * DK + 16 * mt + 4 * lg);
    }
    for (int n = -1; n < N; ++n) {
        const int m = n + 1;
        const bool prep = m < N;
        const bool chain = n >= 0;
        const int cb = (m & 1) ^ 1;     // gate buffer of chunk n
        // ================================ phase 1
        if (chain) {
            // fragment (mr, ks), ks <= mr / 2, in that order; hi and lo parts
            bf16x8 fTU[6], fTUl[6];
#pragma unroll
            for (int mr = 0, f = 0; mr < 4; ++mr)
#pragma unroll
                for (int ks = 0; ks <= mr / 2; ++ks, ++f) {
                    fTU[f] = tfrag<C>(sTU, 16 * mr, ks, lane);
                    fTUl[f] = tfrag<C>(sTUl, 16 * mr, ks, lane);
                }
            // Delta = T diag(beta) Z (the factor's diagonal holds beta)
            f32x4 D[4];
#pragma unroll
            for (int mr = 0, f = 0; mr < 4; ++mr) {
                f32x4 a = zero4(), c = zero4();
#pragma unroll
                for (int ks = 0; ks <= mr / 2; ++ks, ++f) {
                    a = mfma32(fTU[f], zh[ks], a);
                    c = mfma32(fTUl[f], zh[ks], c);
                    a = mfma32(fTU[f], zl[ks], a);
                }
                D[mr] = a + c;
            }
            f32x4 ed[4];   // e^{g_C - g_r} at rows 16 mr + 4 lg + j
#pragma unroll
            for (int mr = 0; mr < 4; ++mr) {
                ed[mr] = ld4(&sG[cb][3][16 * mr + 4 * lg]);
                if constexpr (NQK) ed[mr] = ed[mr] * ld4(&sG[cb][5][16 * mr + 4 * lg]);
            }
            split8(D[0], D[1], sm, dh[0], dl[0]);
            split8(D[2], D[3], sm, dh[1], dl[1]);
            // Delta~ for the state update
            split8(D[0] * ed[0], D[1] * ed[1], sm, th[0], tl[0]);
            split8(D[2] * ed[2], D[3] * ed[3], sm, th[1], tl[1]);
        }
        __syncthreads();
        // ================================ phase 2
        if (chain) {
            // S^T <- e^{g_C} S^T + K^T Delta~
            bf16x8 fk[NMT][2];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) fk[mt][ks] = tfrag<C>(sKT[n & 1], 16 * mt, ks, lane);
            const float egC = sG[cb][1][C - 1];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                st[mt] = st[mt] * egC;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    st[mt] = mfma32(fk[mt][ks], th[ks], st[mt]);
                    st[mt] = mfma32(fk[mt][ks], tl[ks], st[mt]);
                }
            }
            // O = diag(e^g) Q S^T + P Delta (P of chunk n stays in its buffer
            // until phase 2 of the next iteration), stored through a buffer
            // resource covering the valid rows of this chunk (padded rows are
            // dropped).
            bf16x8 fPh[6], fPl[6];   // fragment (mr, ks), ks <= mr / 2, in that order
#pragma unroll
            for (int mr = 0, f = 0; mr < 4; ++mr)
#pragma unroll
                for (int ks = 0; ks <= mr / 2; ++ks, ++f) {
                    fPh[f] = tfrag<C>(sPh, 16 * mr, ks, lane);
                    fPl[f] = tfrag<C>(sPl, 16 * mr, ks, lane);
                }
            const size_t t0 = crow(n);
            const rsrc_t ro = make_rsrc(o + (t0 * H + h) * DV + dv0 + cw,
                                        cvalid(n) * H * DV * (uint32_t)sizeof(TO));
#pragma unroll
            for (int mr = 0; mr < 4; ++mr) {
                const int f = mr < 2 ? mr : 2 * mr - 2;   // first fragment of row tile mr
                f32x4 O = QS[mr];
#pragma unroll
                for (int ks = 0; ks <= mr / 2; ++ks) {
                    O = mfma32(fPh[f + ks], dh[ks], O);
                    O = mfma32(fPl[f + ks], dh[ks], O);
                    O = mfma32(fPh[f + ks], dl[ks], O);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * mr + 4 * lg + j;
                    buf_store(from_f32<TO>(O[j]), ro, (uint32_t)(r * H * DV + lm) * (uint32_t)sizeof(TO));
                }
            }
        }
        if (prep) {
            // hi + lo split of the updated state for the next phase's products
            // (here it overlaps the output products of this phase)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) split8(st[2 * ks], st[2 * ks + 1], sm, sh[ks], sl[ks]);
        }
        __syncthreads();
        // ================================ phase 3
        if (prep) {
            // diag(e^g) Q S^T for chunk m (state now S_m)
            f32x4 eg[4];   // e^{g_r} of chunk m at rows 16 mr + 4 lg + j
#pragma unroll
            for (int mr = 0; mr < 4; ++mr) {
                eg[mr] = ld4(&sG[m & 1][1][16 * mr + 4 * lg]);
                if constexpr (NQK) eg[mr] = eg[mr] * ld4(&sG[m & 1][4][16 * mr + 4 * lg]);
            }
            bf16x8 fq[4][NKS];
#pragma unroll
            for (int mr = 0; mr < 4; ++mr)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) fq[mr][ks] = tfrag<DK>(sQ, 16 * mr, ks, lane);
#pragma unroll
            for (int mr = 0; mr < 4; ++mr) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    acc = mfma32(fq[mr][ks], sh[ks], acc);
                    acc = mfma32(fq[mr][ks], sl[ks], acc);
                }
                QS[mr] = acc * eg[mr];
            }
        }
        if (prep) {
            // Y = K S^T for chunk m from the hi part of S^T, then
            // Z = V - diag(e^g) Y (the V slice of chunk m went to LDS in phase
            // 2; the rows of this lane in the D-order V operand and in the D
            // layout of Y are the same)
            f32x4 Y[4];
            bf16x8 fk[4][NKS];
#pragma unroll
            for (int mr = 0; mr < 4; ++mr)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) fk[mr][ks] = tfrag<DK>(sK, 16 * mr, ks, lane);
#pragma unroll
            for (int mr = 0; mr < 4; ++mr) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) acc = mfma32(fk[mr][ks], sh[ks], acc);
                Y[mr] = acc;
            }
            const bf16x8 fV0 = v_frag(cw / 16, 0);
            const bf16x8 fV1 = v_frag(cw / 16, 1);
            f32x4 Z[4];
#pragma unroll
            for (int mr = 0; mr < 4; ++mr) {
                f32x4 eg = ld4(&sG[m & 1][1][16 * mr + 4 * lg]);
                if constexpr (NQK) eg = eg * ld4(&sG[m & 1][5][16 * mr + 4 * lg]);
                const bf16x8 &fv = mr < 2 ? fV0 : fV1;
#pragma unroll
                for (int j = 0; j < 4; ++j) Z[mr][j] = (float)fv[4 * (mr & 1) + j] - eg[j] * Y[mr][j];
            }
            split8(Z[0], Z[1], sm, zh[0], zl[0]);
            split8(Z[2], Z[3], sm, zh[1], zl[1]);
        }
        __syncthreads();
    }

    if (S_T) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
            *reinterpret_cast<f32x4 *>(S_T + sbase + (size_t)dvw * DK + 16 * mt + 4 * lg) = st[mt];
    }
    // The compiler may join this exit with the producers' entry block; with
    // nothing outstanding here its wait counts in the producer loop stay
    // exact (otherwise the loads above count as pending there, and the
    // producers wait for all their prefetches before each store).
    __builtin_amdgcn_s_waitcnt(0);
}

bool chunk_mfma_supported(int dk, int dv, int chunk) {
    return chunk == kC && dk == dv && (dk == 64 || dk == 128);
}

template <int DK, typename TO, int PRO>
hipError_t launch_chunk_mfma_t(int units, int T, int H, int DV, const int32_t *cu,
                               const void *q, const void *k, const void *v,
                               const float *la, const float *beta, const float *S0,
                               void *o, float *S_T, hipStream_t st) {
    const int ndvt = DV / kDVT;
    const long nwg = (long)units * H * ndvt;
    const int xcd_map = ((long)units * H) % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL((chunk_mfma_kernel<DK, TO, PRO>), dim3((unsigned)nwg), dim3(512), 0, st,
                       T, H, DV, cu != nullptr ? 1 : 0, xcd_map, cu, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)v, la, beta, S0, (TO *)o, S_T);
    return hipGetLastError();
}

hipError_t launch_chunk_mfma(int units, int T, int H, int dk, bool o_bf16, bool norm_qk,
                             bool gates, const int32_t *cu, const void *q, const void *k,
                             const void *v, const float *la, const float *beta,
                             const float *S0, void *o, float *S_T, hipStream_t st) {
    const int pro = (norm_qk ? 1 : 0) | (gates ? 2 : 0);
#define GDN_MFMA_CASE(DKV, TOV, PV)                                                          \
    if (pro == PV)                                                                           \
        return launch_chunk_mfma_t<DKV, TOV, PV>(units, T, H, dk, cu, q, k, v, la, beta, S0, o, \
                                                 S_T, st)
#define GDN_MFMA_TO(DKV, TOV) \
    GDN_MFMA_CASE(DKV, TOV, 0); GDN_MFMA_CASE(DKV, TOV, 1); GDN_MFMA_CASE(DKV, TOV, 2); \
    GDN_MFMA_CASE(DKV, TOV, 3)
#define GDN_MFMA_DK(DKV)                                         \
    if (dk == DKV) {                                             \
        if (o_bf16) { GDN_MFMA_TO(DKV, bf16); } else { GDN_MFMA_TO(DKV, float); } \
    }
    GDN_MFMA_DK(128)
    GDN_MFMA_DK(64)
#undef GDN_MFMA_DK
#undef GDN_MFMA_TO
#undef GDN_MFMA_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
