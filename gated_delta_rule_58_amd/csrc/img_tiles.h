// Operand images shared by the channel-wise decay kernels (KDA, GDN-2): a
// prep launch writes each operand of the sequential launch as a bf16 hi + lo
// pair (hi = x rounded to bf16, lo = bf16(x - hi): about 16 mantissa bits of
// x) with its columns in the order the sequential launch keeps in LDS (rows
// dense in the workspace, padded in LDS); the sequential launch copies it with
// direct global-to-LDS loads and multiplies on the 16x16x32 bf16 MFMA as the
// three piece products hi*hi + lo*hi + hi*lo.
#pragma once

#include "gdn_common.h"

namespace gdn {
namespace img {

// Stored position of column k: within each 32-wide block, lane group g of a
// 16x16x32 MFMA operand takes k = 4g..4g+3 and 16+4g..16+4g+3 (the k order of
// two stacked accumulator tiles), kept together at 8g..8g+7.
__device__ __forceinline__ int dpos(int k) {
    return (k & ~31) + ((k & 16) >> 2) + 2 * (k & 12) + (k & 3);
}

// Four consecutive values as hi and lo bf16 (8-byte stores).
__device__ __forceinline__ void put_pair4(bf16 *hi, bf16 *lo, f32x4 x) {
    bf16x4 h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = (bf16)x[j];
        l[j] = (bf16)(x[j] - (float)h[j]);
    }
    *reinterpret_cast<bf16x4 *>(hi) = h;
    *reinterpret_cast<bf16x4 *>(lo) = l;
}
// Eight values (D-order group: two runs of four) as hi and lo bf16 (16-byte stores).
__device__ __forceinline__ void put_pair8(bf16 *hi, bf16 *lo, f32x4 x0, f32x4 x1) {
    bf16x8 h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = (bf16)x0[j];
        l[j] = (bf16)(x0[j] - (float)h[j]);
        h[4 + j] = (bf16)x1[j];
        l[4 + j] = (bf16)(x1[j] - (float)h[4 + j]);
    }
    *reinterpret_cast<bf16x8 *>(hi) = h;
    *reinterpret_cast<bf16x8 *>(lo) = l;
}
__device__ __forceinline__ void put_pair1(bf16 *hi, bf16 *lo, float x) {
    const bf16 h = (bf16)x;
    *hi = h;
    *lo = (bf16)(x - (float)h);
}

__device__ __forceinline__ bf16x8 ld8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// A region of operand images whose rows are padded by 8 bf16 (one 16-byte
// chunk) in LDS but dense in the workspace: M x R rows of W bf16, then E
// more 16-byte chunks (stored alike in both), then the tail of the region's
// whole KB in LDS.  src_chunk(q) is the chunk of the dense image that LDS
// chunk q holds; a row's pad chunk and the tail read chunk 0 (never read
// back from LDS), so every source address lies inside the image.
template <int M, int R, int W, int E> struct PaddedRegion {
    static constexpr int DC = W / 8, PC = DC + 1, NM = M * R * PC;
    static_assert(W % 8 == 0, "whole 16-byte chunks per row");
    __device__ static __forceinline__ int src_chunk(int q) {
        if (q < NM) {
            const int row = q / PC, ch = q - row * PC;
            return row * DC + (ch < DC ? ch : 0);
        }
        return q < NM + E ? M * R * DC + (q - NM) : 0;
    }
};

// Stores of output rows through a raw buffer resource whose size covers only
// the valid rows of a chunk: stores past them (ragged last chunk) are dropped
// by the hardware range check, so no lane branches on the row.  The base
// address must be wave-uniform; lanes differ by their byte offsets.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t rows_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);   // raw, 32-bit data format
}
__device__ __forceinline__ void rsrc_store(float x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, off, 0, 0);
}
__device__ __forceinline__ void rsrc_store(bf16 x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, off, 0, 0);
}

// Direct global-to-LDS copy of 16 bytes per lane: lane l's bytes land at
// dst + 16 l (dst is the wave's base address), so a wave moves 1 KB.
__device__ __forceinline__ void lds_dma16(void *dst, const void *src) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// s_waitcnt vmcnt(N): wait until at most N of this wave's vector memory
// operations are outstanding (they complete in issue order).
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace img
}  // namespace gdn
