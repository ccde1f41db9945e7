// Host-only stand-ins for the kernel launchers of libgdn.so, so that the C
// ABI's validation code (csrc/abi.cpp) can be built with the address and
// undefined-behaviour sanitizers and run without a GPU.  Each launcher
// records that it was reached and returns success; the support predicates
// accept the instances the real kernels are compiled for; the workspace
// sizes follow the real per-chunk-and-head sizes closely enough for the
// size checks to be exercised.
#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>

int g_launches = 0;

namespace gdn {
static hipError_t reached() { ++g_launches; return hipSuccess; }
hipError_t launch_step(int, int, int, int, bool, bool, bool, bool, const void *, const void *,
                       const void *, const float *, const float *, float *, void *,
                       hipStream_t) { return reached(); }
bool chunk_f32_supported(int dk, int dv, int chunk) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64) &&
           (chunk == 16 || chunk == 32 || chunk == 64);
}
hipError_t launch_chunk_f32(int, int, int, int, int, bool, bool, bool, const int32_t *,
                            const void *, const void *, const void *, const float *,
                            const float *, const float *, void *, float *, hipStream_t) {
    return reached();
}
bool chunk_mfma_supported(int dk, int dv, int chunk) {
    return chunk == 64 && dk == dv && (dk == 64 || dk == 128);
}
hipError_t launch_chunk_mfma(int, int, int, int, bool, bool, bool, const int32_t *, const void *,
                             const void *, const void *, const float *, const float *,
                             const float *, void *, float *, hipStream_t) { return reached(); }
bool chunk_bwd_supported(int dk, int dv, int chunk, bool bf) {
    return chunk == 64 && dk == dv && (bf ? (dk == 64 || dk == 128) : dk == 64);
}
size_t chunk_bwd_ws_bytes(int units, int T, int H, int d, bool) {
    return (size_t)(units + T / 64 + 1) * (size_t)H * (2 * 64 * 64 + 3 * 64 * d + d + 64) * 4;
}
hipError_t launch_chunk_bwd(int, int, int, int, bool, bool, const int32_t *, const void *,
                            const void *, const void *, const float *, const float *,
                            const float *, const void *, const float *, void *, void *, void *,
                            float *, float *, float *, void *, hipStream_t) { return reached(); }
bool kda_supported(int dk, int dv, int chunk, bool bf) { return chunk_bwd_supported(dk, dv, chunk, bf); }
size_t kda_ws_bytes(int units, int T, int H, int d, bool v) { return chunk_bwd_ws_bytes(units, T, H, d, v); }
size_t kda_scratch_bytes() { return size_t(64) << 20; }
static unsigned char g_fake_scratch[256];
hipError_t kda_scratch_ptr(void **ptr) { *ptr = g_fake_scratch; return hipSuccess; }
hipError_t launch_kda_fwd(int, int, int, int, bool, bool, const int32_t *, const void *,
                          const void *, const void *, const float *, const float *, const float *,
                          void *, float *, void *, hipStream_t) { return reached(); }
bool gdn2_supported(int dk, int dv, int chunk, bool bf) { return chunk_bwd_supported(dk, dv, chunk, bf); }
size_t gdn2_ws_bytes(int units, int T, int H, int d, bool v) { return chunk_bwd_ws_bytes(units, T, H, d, v); }
hipError_t launch_gdn2_fwd(int, int, int, int, bool, bool, const int32_t *, const void *,
                           const void *, const void *, const float *, const float *,
                           const float *, const float *, void *, float *, void *,
                           hipStream_t) { return reached(); }
}  // namespace gdn
