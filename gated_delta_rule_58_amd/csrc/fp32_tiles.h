// fp32-MFMA tile helpers shared by the backward and the channel-wise decay
// kernels: 64-token chunks, 16 x 16 fp32 tiles on v_mfma_f32_16x16x4_f32
// (lane l supplies A[l & 15][l >> 4] and B[l >> 4][l & 15] and holds
// D[4 (l >> 4) + j][l & 15], j = 0..3), chunk-slot geometry, gate scans and
// 16-byte staging copies.
#pragma once

#include "gdn_common.h"

namespace gdn {
namespace tiles {

constexpr int BC = 64;         // chunk length
constexpr int LDN = BC + 4;    // row stride (floats) of 64 x 64 fp32 LDS matrices

// Row stride (elements) of a 64 x D LDS matrix of type X: 4 floats or 8
// bf16 of padding put consecutive rows 4 banks apart.
template <typename X, int D> constexpr int ldx() { return sizeof(X) == 2 ? D + 8 : D + 4; }

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc[t] += sum_{k < K} A(i, k) B_t(k, j) on NT 16 x 16 tiles side by side,
// with A(i, k) = A[i * ar + k * ak] and B_t(k, j) = B[t * bt + k * bk + j * bj]
// (pointers at the tiles' origin, any layout).  Lane (i = l & 15, q = l >> 4)
// ends with rows 4q..4q+3 of column i.  One A read per k step feeds NT
// independent accumulation chains.
template <int K, int NT, typename TA, typename TB>
__device__ __forceinline__ void mmn(const TA *A, int ar, int ak, const TB *B, int bk, int bj,
                                    int bt, f32x4 (&acc)[NT], int lane) {
    const int i = lane & 15, q = lane >> 4;
    const TA *pa = A + i * ar + q * ak;
    const TB *pb = B + q * bk + i * bj;
#pragma unroll 4
    for (int k = 0; k < K; k += 4) {
        const float a = to_f32(pa[k * ak]);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = mfma_f32(a, to_f32(pb[t * bt + k * bk]), acc[t]);
    }
}
template <int NT> __device__ __forceinline__ void zero_n(f32x4 (&acc)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = zero4();
}

// Lane data moved by DPP (all lanes active): quad permutations and row mirrors.
template <int CTRL> __device__ __forceinline__ float dppf(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a row group, in every lane: the partner of each
// step is lane ^ 1, lane ^ 2 (quad permutations), the other quad of the
// half-row, the other half-row (mirrors) -- the same pairs of partial sums as
// a butterfly over lane ^ 1, ^ 2, ^ 4, ^ 8, without a trip through LDS.
__device__ __forceinline__ float sum16(float x) {
    x += dppf<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dppf<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dppf<0x141>(x);   // row_half_mirror
    x += dppf<0x140>(x);   // row_mirror
    return x;
}
// x + x[lane ^ 16], then the same with lane ^ 32: a sum over the four row
// groups, in every lane (gfx950 permlane swaps; each sum adds the same two
// values in every lane, as the butterfly does).
__device__ __forceinline__ float sum_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Maximum over the 64 lanes of a wave, in every lane: the butterfly of
// sum16 and sum_rows with fmaxf.
__device__ __forceinline__ float max64(float x) {
    x = fmaxf(x, dppf<0xB1>(x));
    x = fmaxf(x, dppf<0x4E>(x));
    x = fmaxf(x, dppf<0x141>(x));
    x = fmaxf(x, dppf<0x140>(x));
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename X> __device__ __forceinline__ X cvt(float x);
template <> __device__ __forceinline__ float cvt<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 cvt<bf16>(float x) { return (bf16)x; }

// --- chunk geometry -------------------------------------------------------
// Chunk slots: a dense batch has NC = ceil(T / 64) slots per sequence,
// sequence u starting at slot u NC; packed sequences start at slot
// floor(cu[u] / 64) + u, which leaves room for every sequence's
// ceil(L / 64) chunks (slots between sequences stay unused).
__device__ __forceinline__ int unit_base(int u, int NC, int varlen, const int32_t *cu) {
    return varlen ? cu[u] / BC + u : u * NC;
}

__device__ __forceinline__ void unit_span(int u, int T, int varlen, const int32_t *cu,
                                          long &start, long &L) {
    if (varlen) {
        start = cu[u];
        L = (long)cu[u + 1] - cu[u];
    } else {
        start = (long)u * T;
        L = T;
    }
}

// Slot -> (first token, valid rows); false for an unused slot.
__device__ __forceinline__ bool slot_chunk(int slot, int units, int T, int NC, int varlen,
                                           const int32_t *cu, long &row0, int &n) {
    if (!varlen) {
        const int u = slot / NC, c = slot % NC;
        if (u >= units) return false;
        row0 = (long)u * T + (long)c * BC;
        n = min(BC, T - c * BC);
        return true;
    }
    int lo = 0, hi = units - 1;   // largest u with base(u) <= slot (base(0) = 0)
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] / BC + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int c = slot - (cu[lo] / BC + lo);
    const long L = (long)cu[lo + 1] - cu[lo];
    if ((long)c * BC >= L) return false;
    row0 = cu[lo] + (long)c * BC;
    n = (int)min((long)BC, L - (long)c * BC);
    return true;
}

// Gates of one chunk, by one wave: sg[0] = g (chunk-local prefix of log
// alpha; padded tokens add 0), sg[1] = e^g, sg[2] = beta (0 when padded),
// sg[3] = e^{g_n - g} with g_n the prefix at the last valid token.
__device__ __forceinline__ void chunk_gates(float (*sg)[BC], const float *la, const float *beta,
                                            long row0, int n, int H, int h, int lane) {
    float x = 0.f, b = 0.f;
    if (lane < n) {
        const size_t idx = (size_t)(row0 + lane) * H + h;
        x = la[idx];
        b = beta[idx];
    }
    x = wave_scan64(x);
    const float gn = lane63(x);
    sg[0][lane] = x;
    sg[1][lane] = expf(x);
    sg[2][lane] = b;
    sg[3][lane] = expf(gn - x);
}

// 16-byte vector copies between global memory and LDS.  Every row start
// used below is 16-byte aligned: global rows are d_k or d_v elements of a
// 16-byte aligned tensor, LDS rows are padded to multiples of 16 bytes.
__device__ __forceinline__ void put8(float *dst, bf16x8 x) {
    *reinterpret_cast<f32x4 *>(dst) = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{(float)x[4], (float)x[5], (float)x[6], (float)x[7]};
}
__device__ __forceinline__ void put8(bf16 *dst, bf16x8 x) { *reinterpret_cast<bf16x8 *>(dst) = x; }
__device__ __forceinline__ void put4(float *dst, f32x4 x) { *reinterpret_cast<f32x4 *>(dst) = x; }

// Rows [row0, row0 + n) of a [tokens, H, D] tensor, columns col0..col0+width,
// into a 64-row LDS matrix (row stride ld); rows n..63 are zero.
template <int D, typename TS, typename TG>
__device__ __forceinline__ void load_rows(TS *dst, int ld, const TG *src, long row0, int n, int H,
                                          int h, int col0, int width, int tid, int nthr) {
    constexpr int V = sizeof(TG) == 2 ? 8 : 4;   // elements per 16-byte load
    const int per_row = width / V;
    for (int e = tid; e < BC * per_row; e += nthr) {
        const int r = e / per_row, c = (e % per_row) * V;
        TS *d = dst + r * ld + c;
        const TG *sp = src + ((size_t)(row0 + r) * H + h) * D + col0 + c;
        if constexpr (V == 8) {
            bf16x8 x = {};
            if (r < n) x = *reinterpret_cast<const bf16x8 *>(sp);
            put8(d, x);
        } else {
            f32x4 x = zero4();
            if (r < n) x = *reinterpret_cast<const f32x4 *>(sp);
            if constexpr (sizeof(TS) == 4) {
                put4(reinterpret_cast<float *>(d), x);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] = cvt<TS>(x[j]);
            }
        }
    }
}
// Rows of a [64, D] fp32 workspace block (rows >= n are zero).
template <int D>
__device__ __forceinline__ void load_ws_rows(float *dst, int ld, const float *src, int n, int tid,
                                             int nthr) {
    for (int e = tid; e < BC * D / 4; e += nthr) {
        const int r = e / (D / 4), c = (e % (D / 4)) * 4;
        f32x4 x = zero4();
        if (r < n) x = *reinterpret_cast<const f32x4 *>(src + (size_t)r * D + c);
        put4(dst + r * ld + c, x);
    }
}
__device__ __forceinline__ void put4(bf16 *dst, f32x4 x) {
    *reinterpret_cast<bf16x4 *>(dst) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

template <typename X> struct Vec16;
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };

// A 64-row block (W elements per row, rows >= n zero) fetched into registers
// by a 512-thread workgroup, 16 bytes at a time, and written to LDS later:
// the sequential kernels fetch the next chunk's operands while they work on
// the current one.
template <int W, typename TG> struct Prefetch {
    typedef typename Vec16<TG>::type VT;
    static constexpr int V = Vec16<TG>::n, PR = W / V, NP = (BC * PR + 511) / 512;
    VT buf[NP];
    __device__ __forceinline__ void fetch(const TG *src, size_t row_stride, int n, int tid) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int e = tid + 512 * i, r = e / PR, c = (e % PR) * V;
            buf[i] = VT{};
            if (e < BC * PR && r < n) buf[i] = *reinterpret_cast<const VT *>(src + r * row_stride + c);
        }
    }
    template <typename TS> __device__ __forceinline__ void commit(TS *dst, int ld, int tid) const {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int e = tid + 512 * i, r = e / PR, c = (e % PR) * V;
            if (e < BC * PR) {
                if constexpr (V == 8) put8(dst + r * ld + c, buf[i]);
                else put4(dst + r * ld + c, buf[i]);
            }
        }
    }
};

// The chunk's log alpha and beta for lane `lane` of one wave (0 past n),
// then the scan that chunk_gates does.
__device__ __forceinline__ void gate_fetch(const float *la, const float *beta, long row0, int n,
                                           int H, int h, int lane, float &x, float &b) {
    x = 0.f;
    b = 0.f;
    if (lane < n) {
        const size_t idx = (size_t)(row0 + lane) * H + h;
        x = la[idx];
        b = beta[idx];
    }
}
__device__ __forceinline__ void gate_scan(float (*sg)[BC], float x, float b, int lane) {
    x = wave_scan64(x);
    const float gn = lane63(x);
    sg[0][lane] = x;
    sg[1][lane] = expf(x);
    sg[2][lane] = b;
    sg[3][lane] = expf(gn - x);
}

// Zero the six 16 x 16 blocks above the diagonal of a 64 x 64 fp32 LDS
// matrix (row stride LDN), one 16-byte store per item: the rest of such a
// matrix is written whole (its diagonal blocks masked) before it is read.
__device__ __forceinline__ void zero_upper(float *m, int tid) {
    for (int e = tid; e < 6 * 64; e += 512) {
        const int blk = e >> 6, w = e & 63;   // blocks (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
        const int rb = blk < 3 ? 0 : blk < 5 ? 1 : 2, cb = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
        *reinterpret_cast<f32x4 *>(m + (16 * rb + (w >> 2)) * LDN + 16 * cb + 4 * (w & 3)) = zero4();
    }
}

// In-place prefix over the BC rows of each of the D columns of an fp32 LDS
// tile (row stride ld), by all 512 threads (every lane must call it): column
// c = tid / SEG is cut into SEG = 512 / D segments of rows, lane tid % SEG
// sums its segment in registers, and the segment totals are combined across
// the SEG lanes of the column by shuffles.  Each thread rewrites only the
// elements it read.  Returns the column's total (the prefix at the last row)
// in every lane of the column's group.  Each element is multiplied by
// `scale` as it is read (a change of units, e.g. to base-2 exponents).
template <int D> __device__ __forceinline__ float column_prefix(float *s, int ld, int tid, float scale = 1.f) {
    constexpr int SEG = 512 / D, RS = BC / SEG;
    static_assert(SEG * D == 512 && RS * SEG == BC, "512 threads cover the tile");
    const int c = tid / SEG, sg = tid % SEG;
    float *col = s + sg * RS * ld + c;
    float v[RS];
#pragma unroll
    for (int j = 0; j < RS; ++j) v[j] = col[j * ld] * scale;
#pragma unroll
    for (int j = 1; j < RS; ++j) v[j] += v[j - 1];
    float incl = v[RS - 1];   // inclusive scan of the segment totals
#pragma unroll
    for (int o = 1; o < SEG; o <<= 1) {
        const float y = __shfl_up(incl, o, SEG);
        if (sg >= o) incl += y;
    }
    float off = __shfl_up(incl, 1, SEG);
    off = sg > 0 ? off : 0.f;
#pragma unroll
    for (int j = 0; j < RS; ++j) col[j * ld] = v[j] + off;
    return __shfl(incl, SEG - 1, SEG);
}

__device__ __forceinline__ void load_nn(float *dst, const float *src, int tid, int nthr) {
    for (int e = tid; e < BC * BC / 4; e += nthr)
        put4(dst + (e >> 4) * LDN + (e & 15) * 4, *reinterpret_cast<const f32x4 *>(src + 4 * e));
}

// Lane S of each group of four lanes, to all four (DPP quad permutation).
template <int S> __device__ __forceinline__ float quad_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), S * 0x55, 0xf, 0xf, false));
}

// T = (I + A)^{-1} for a strictly lower 64 x 64 A in LDS (row stride LDN;
// only its diagonal and lower blocks are read) into X (row stride LDN; the
// diagonal and lower blocks are written whole, the caller zeroes the blocks
// above), by all 512 threads of the workgroup (it contains workgroup
// barriers): the four 16 x 16 diagonal
// blocks by forward substitution in registers (wave b inverts block b), then
// the blocks below the diagonal level by level,
// T_ij = -T_ii sum_{j <= k < i} A_ik T_kj, on MFMA.
//
// Diagonal block: lane (column cl = lane / 4, row group q = lane % 4) holds
// rows 4q..4q+3 of column cl of the block's inverse.  The four row groups are
// solved in order: group s solves its 4 x 4 unit lower system, its rows are
// broadcast to the other lanes of the quad (same column) by DPP, and the
// later groups subtract their rows' share of them.
__device__ __forceinline__ void block_inverse64(const float *sA, float *sX, int wave, int lane) {
    if (wave < 4) {
        const int b = wave, cl = lane >> 2, q = lane & 3;
        const float *Ab = sA + 16 * b * LDN + 16 * b;
        f32x4 x;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) x[rr] = (4 * q + rr == cl) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            f32x4 acol[4];   // acol[k][rr] = A_bb[4 q + rr][4 s + k]
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 row = *reinterpret_cast<const f32x4 *>(Ab + (4 * q + rr) * LDN + 4 * s);
#pragma unroll
                for (int k = 0; k < 4; ++k) acol[k][rr] = row[k];
            }
            f32x4 t = x;   // group s: rows 4 s .. 4 s + 3, unit lower 4 x 4 solve
#pragma unroll
            for (int c = 0; c < 3; ++c)
#pragma unroll
                for (int rr = c + 1; rr < 4; ++rr) t[rr] -= acol[c][rr] * t[c];
            const bool mine = q == s, later = q > s;   // lane-varying: selects, not branches
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) x[rr] = mine ? t[rr] : x[rr];
            if (s < 3) {
                f32x4 xb;   // the solved rows 4 s .. 4 s + 3 of this column
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    xb[k] = s == 0 ? quad_bcast<0>(x[k]) : s == 1 ? quad_bcast<1>(x[k]) : quad_bcast<2>(x[k]);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float y = x[rr] - ((acol[0][rr] * xb[0] + acol[1][rr] * xb[1]) +
                                             (acol[2][rr] * xb[2] + acol[3][rr] * xb[3]));
                    x[rr] = later ? y : x[rr];
                }
            }
        }
        float *Xb = sX + 16 * b * LDN + 16 * b;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Xb[(4 * q + rr) * LDN + cl] = x[rr];
    }
    __syncthreads();
#pragma unroll
    for (int lev = 1; lev < 4; ++lev) {
        if (wave < 4 - lev) {
            const int jb = wave, ib = wave + lev;   // block (ib, jb)
            f32x4 m[1];
            zero_n(m);
            for (int kb = jb; kb < ib; ++kb)
                mmn<16, 1>(sA + 16 * ib * LDN + 16 * kb, LDN, 1, sX + 16 * kb * LDN + 16 * jb, LDN,
                           1, 0, m, lane);
            float *blk = sX + 16 * ib * LDN + 16 * jb;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) blk[(4 * (lane >> 4) + jj) * LDN + (lane & 15)] = m[0][jj];
            __builtin_amdgcn_wave_barrier();
            f32x4 t[1];
            zero_n(t);
            mmn<16, 1>(sX + 16 * ib * LDN + 16 * ib, LDN, 1, blk, LDN, 1, 0, t, lane);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) blk[(4 * (lane >> 4) + jj) * LDN + (lane & 15)] = -t[0][jj];
        }
        __syncthreads();
    }
}

// Four consecutive elements (8- or 16-byte aligned) as floats.
__device__ __forceinline__ f32x4 ld4f(const bf16 *p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ f32x4 ld4f(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// acc1[t] += A1 B_t^T and acc2[t] += A2 B_t^T for fp32 operands read by
// rows from LDS (pointers at the tiles' first rows, row strides lda and ldb,
// 16-byte aligned; tile t of B starts 16 t rows down).  Lane (li, lq) reads
// the 4 consecutive k values 16 s + 4 lq .. + 3 of its row in one 16-byte
// read, so the k order of each MFMA step is the same for both operands, and
// the two products share the B reads.
template <int K, int NT>
__device__ __forceinline__ void mm_rows2(const float *A1, const float *A2, int lda, const float *B,
                                         int ldb, f32x4 (&acc1)[NT], f32x4 (&acc2)[NT], int lane) {
    const int li = lane & 15, lq = lane >> 4;
    const float *pa1 = A1 + li * lda + 4 * lq, *pa2 = A2 + li * lda + 4 * lq;
    const float *pb = B + li * ldb + 4 * lq;
#pragma unroll 2
    for (int s = 0; s < K / 16; ++s) {
        const f32x4 a1 = ld4f(pa1 + 16 * s), a2 = ld4f(pa2 + 16 * s);
        f32x4 b[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) b[t] = ld4f(pb + 16 * t * ldb + 16 * s);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc1[t] = mfma_f32(a1[m], b[t][m], acc1[t]);
                acc2[t] = mfma_f32(a2[m], b[t][m], acc2[t]);
            }
    }
}

// Diagonal 16 x 16 block b of the channel-weighted product
//   M[r][i] = sum_c X[r][c] Y[i][c] e^{G[r][c] - G[i][c]},  r, i in 16b..16b+15,
// by one wave, every entry (the caller masks the upper part); lane (li, lq)
// gets rows 16b + 4lq + j of column 16b + li.  G is the chunk's per-channel
// prefix (non-increasing down the rows).  With G_ref the prefix just before
// the block (0 for the first), the weight factors as e^{G_r - G_ref} (<= 1)
// times e^{G_ref - G_i} (>= 1): when the block's span max_c (G_ref - G_last)
// is at most 60 both factors are normal floats and the block is one MFMA
// product; otherwise it is formed term by term (exponentials of r >= i only).
// Decay span max_c (G_ref - G_last) of diagonal block b (all lanes get it).
template <int D>
__device__ __forceinline__ float diag_span(const float *G, int lg, int b, int lane) {
    const float *gref = b > 0 ? G + (16 * b - 1) * lg : nullptr;
    const float *glast = G + (16 * b + 15) * lg;
    float span = 0.f;
    for (int c = lane; c < D; c += 64) span = fmaxf(span, (gref ? gref[c] : 0.f) - glast[c]);
    return max64(span);
}
// The same block term by term (exponentials of r >= i only), for any span;
// with BASE2 the prefixes G are in base-2 units (log2 e times the natural).
template <int D, bool BASE2 = false, typename TX, typename TY>
__device__ __forceinline__ f32x4 diag_terms(const TX *X, int lx, const TY *Y, int ly,
                                            const float *G, int lg, int b, int lane) {
    const int li = lane & 15, lq = lane >> 4;
    f32x4 acc = zero4();
    const int i = 16 * b + li;
    for (int c = 0; c < D; c += 4) {
        const f32x4 gi = *reinterpret_cast<const f32x4 *>(G + i * lg + c);
        const f32x4 yi = ld4f(Y + i * ly + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * b + 4 * lq + j;
            const f32x4 gr = *reinterpret_cast<const f32x4 *>(G + r * lg + c);
            const f32x4 xr = ld4f(X + r * lx + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = fminf(gr[e] - gi[e], 0.f);
                acc[j] += xr[e] * yi[e] * (BASE2 ? __builtin_amdgcn_exp2f(x) : __expf(x));
            }
        }
    }
    return acc;
}
// (BASE2: the prefixes G in base-2 units, as for diag_terms.)
template <int D, bool BASE2 = false, typename TX, typename TY>
__device__ __forceinline__ f32x4 diag_block(const TX *X, int lx, const TY *Y, int ly,
                                            const float *G, int lg, int b, int lane) {
    const int li = lane & 15, lq = lane >> 4;
    constexpr float kSpan = BASE2 ? 60.f * 1.4426950408889634f : 60.f;
    if (diag_span<D>(G, lg, b, lane) > kSpan) return diag_terms<D, BASE2>(X, lx, Y, ly, G, lg, b, lane);
    auto ex = [](float x) { return BASE2 ? __builtin_amdgcn_exp2f(x) : __expf(x); };
    const float gon = b > 0 ? 1.f : 0.f;   // reference prefix 0 for the first block
    const float *gref = G + (b > 0 ? 16 * b - 1 : 0) * lg;
    f32x4 acc = zero4();
    const int rw = 16 * b + li;
    // step j of channel group c0: lane (li, lq) supplies channel c0 + 4 lq + j
#pragma unroll 2
    for (int c0 = 0; c0 < D; c0 += 16) {
        const int cb = c0 + 4 * lq;
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(gref + cb) * gon;
        const f32x4 gw = *reinterpret_cast<const f32x4 *>(G + rw * lg + cb);
        const f32x4 xa = ld4f(X + rw * lx + cb), ya = ld4f(Y + rw * ly + cb);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc = mfma_f32(xa[j] * ex(gw[j] - gr[j]), ya[j] * ex(gr[j] - gw[j]), acc);
    }
    return acc;
}

}  // namespace tiles
}  // namespace gdn
