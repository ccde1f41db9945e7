// Shared device helpers of the gfx950 gated-delta-rule kernels: bf16
// conversion, the 16x16 MFMA fragment layouts and LDS fragment loaders.
//
// MFMA conventions (v_mfma_f32_16x16x32_bf16, wave64):
//   A operand (16 x 32): lane l holds 8 k-values of row (l & 15);
//   B operand (32 x 16): lane l holds 8 k-values of column (l & 15);
//   D / C (16 x 16 fp32): lane l holds rows 4*(l >> 4) + j, j = 0..3, of
//   column (l & 15).
// Which 8 k-values a lane holds only has to agree between A and B, so two
// k-orders are used:
//   natural  -- lane group g = l >> 4 holds k = 8g .. 8g+7;
//   "D-order" -- group g holds k = 4g .. 4g+3 and 16+4g .. 16+4g+3, which is
//   exactly what two stacked D tiles hold.  A matrix produced by an MFMA in
//   D layout can therefore feed the next MFMA as a B operand (or, if the
//   transposed product was computed, as an A operand) straight from
//   registers; the other operand is then read from LDS in D-order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16x16x32 bf16 MFMA, fp32 accumulate: acc += A * B.
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// 16x16x16 bf16 MFMA: lane l holds A[l&15][4(l>>4)..+3], B[4(l>>4)..+3][l&15].
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Round two D tiles (rows 0-15 and 16-31 of a 32-row block) to a bf16
// operand in D-order.
__device__ __forceinline__ bf16x8 d_to_op(f32x4 d0, f32x4 d1) {
    return bf16x8{(bf16)d0[0], (bf16)d0[1], (bf16)d0[2], (bf16)d0[3],
                  (bf16)d1[0], (bf16)d1[1], (bf16)d1[2], (bf16)d1[3]};
}

// Split x into hi + lo, both bf16: hi = bf16(x) (round to nearest even),
// lo = bf16(x - hi).  x - (hi + lo) is below 2^-16 |x|, so products
// hi*y + lo*y keep about 16 mantissa bits of x, and hi alone is x rounded
// to bf16.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo) {
    typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
    hi = __builtin_bit_cast(uint32_t, bf16x2{(bf16)a, (bf16)b});
    const float ha = __builtin_bit_cast(float, hi << 16);
    const float hb = __builtin_bit_cast(float, hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, bf16x2{(bf16)(a - ha), (bf16)(b - hb)});
}
__device__ __forceinline__ void split_op(f32x4 d0, f32x4 d1, bf16x8 &hi, bf16x8 &lo) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split_pair(d0[0], d0[1], h0, l0);
    split_pair(d0[2], d0[3], h1, l1);
    split_pair(d1[0], d1[1], h2, l2);
    split_pair(d1[2], d1[3], h3, l3);
    hi = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
}

// --- LDS fragment loaders (row-major bf16 arrays with `ld` elements/row) ---

// Rows row0..row0+15, k0..k0+31 in natural order: one 16-byte read.
__device__ __forceinline__ bf16x8 frag_rows(const bf16 *base, int ld, int row0,
                                            int k0, int lane) {
    return *reinterpret_cast<const bf16x8 *>(base + (row0 + (lane & 15)) * ld + k0 +
                                             8 * (lane >> 4));
}

// Rows row0..row0+15, k0..k0+31 in D-order: two 8-byte reads.
__device__ __forceinline__ bf16x8 frag_rows_d(const bf16 *base, int ld, int row0,
                                              int k0, int lane) {
    const bf16 *p = base + (row0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    return cat(*reinterpret_cast<const bf16x4 *>(p),
               *reinterpret_cast<const bf16x4 *>(p + 16));
}

// Transposed access: operand element (m, k) = X[k0 + k][m0 + m] of a
// row-major X, natural k order (8 two-byte reads).
__device__ __forceinline__ bf16x8 frag_cols(const bf16 *base, int ld, int m0,
                                            int k0, int lane) {
    const bf16 *p = base + (k0 + 8 * (lane >> 4)) * ld + m0 + (lane & 15);
    bf16x8 r;
#pragma unroll
    for (int s = 0; s < 8; ++s) r[s] = p[s * ld];
    return r;
}

// Transposed access in D-order.
__device__ __forceinline__ bf16x8 frag_cols_d(const bf16 *base, int ld, int m0,
                                              int k0, int lane) {
    const bf16 *p = base + (k0 + 4 * (lane >> 4)) * ld + m0 + (lane & 15);
    bf16x8 r;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        r[s] = p[s * ld];
        r[4 + s] = p[(16 + s) * ld];
    }
    return r;
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active) by
// DPP: row shifts by 1, 2, 4 and 8 scan each row of 16 lanes (lanes without
// a source add 0), then the last lane of rows 0 and 2 is added to rows 1 and
// 3, then lane 31 to rows 2 and 3.
template <int CTRL, int ROWS> __device__ __forceinline__ float dpp_add_src(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_scan64(float x) {
    x += dpp_add_src<0x111, 0xf>(x);   // row_shr:1
    x += dpp_add_src<0x112, 0xf>(x);   // row_shr:2
    x += dpp_add_src<0x114, 0xf>(x);   // row_shr:4
    x += dpp_add_src<0x118, 0xf>(x);   // row_shr:8
    x += dpp_add_src<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_add_src<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}
// The value of lane 63 (wave-uniform).
__device__ __forceinline__ float lane63(float x) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// LDS transpose read of 16-bit elements (gfx950 ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane 4j + q passes the address of 4 consecutive
// elements (8 bytes); lane i of the group gets, as its element j, element i % 4
// of the 8 bytes addressed by lane 4j + i / 4.  So if lane 4j + q points at
// row r_j, columns c0 + 4q .. c0 + 4q + 3 of a row-major matrix, lane i gets
// column c0 + i of rows r_0..r_3: a column gather in one instruction.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16 *p) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)p));
}

}  // namespace gdn
