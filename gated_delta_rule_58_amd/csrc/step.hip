// Recurrent decode step of the gated delta rule on gfx950.
//
// One token per (b, h): with the current read p = S k, the rule
//   S' = alpha S + (beta v - alpha beta p) k^T,   o = S' q
// ("Gated Delta Networks: Improving Mamba2 with Delta Rule", research-map
// summary, section "Approach", multiplied out; read-out on the updated
// state).  Since o = S' q = alpha (S q) + u (k . q) with u = beta (v - alpha p),
// each row of S is read once, both dot products come from that single read,
// and the row is written back once: the kernel streams the fp32 state at the
// HBM rate and does no other memory traffic worth counting.
//
// Mapping: 16 lanes own one row of S (d_k/16 consecutive floats each, so a
// row is one contiguous 256/512-byte access); a 256-thread workgroup covers
// 32 rows of one (b, h) in two passes whose loads are issued together.
#include "gdn_common.h"

namespace gdn {

constexpr int kStepRowsPerWG = 32;

template <int N, typename TI>
__device__ __forceinline__ void load_vec(const TI *p, float (&r)[N]);

template <>
__device__ __forceinline__ void load_vec<8, bf16>(const bf16 *p, float (&r)[8]) {
    bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (float)x[i];
}
template <>
__device__ __forceinline__ void load_vec<4, bf16>(const bf16 *p, float (&r)[4]) {
    bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (float)x[i];
}
template <>
__device__ __forceinline__ void load_vec<8, float>(const float *p, float (&r)[8]) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
}
template <>
__device__ __forceinline__ void load_vec<4, float>(const float *p, float (&r)[4]) {
    float4 a = *reinterpret_cast<const float4 *>(p);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
}

__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 8, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 1, 16);
    return x;
}

template <int DK, typename TI, typename TO>
__global__ __launch_bounds__(256) void step_kernel(
    int DV, const TI *__restrict__ q, const TI *__restrict__ k,
    const TI *__restrict__ v, const float *__restrict__ log_alpha,
    const float *__restrict__ beta, float *__restrict__ S, TO *__restrict__ o) {
    constexpr int VEC = DK / 16;   // floats of a row per lane
    constexpr int NV4 = VEC / 4;
    constexpr int NP = 2;          // passes of 4 rows per wave
    const int unit = blockIdx.x;   // b * H + h
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 15;

    float kr[VEC], qr[VEC];
    load_vec<VEC, TI>(k + (size_t)unit * DK + c * VEC, kr);
    load_vec<VEC, TI>(q + (size_t)unit * DK + c * VEC, qr);
    const float a = expf(log_alpha[unit]);
    const float b = beta[unit];

    int row[NP];
    float4 s[NP][NV4];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        row[p] = blockIdx.y * kStepRowsPerWG + wave * (4 * NP) + p * 4 + (lane >> 4);
        if (row[p] < DV) {
            const float4 *sp = reinterpret_cast<const float4 *>(
                S + ((size_t)unit * DV + row[p]) * DK + c * VEC);
#pragma unroll
            for (int i = 0; i < NV4; ++i) s[p][i] = sp[i];
        }
    }

    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) kq += kr[i] * qr[i];
    kq = sum16(kq);

#pragma unroll
    for (int p = 0; p < NP; ++p) {
        if (row[p] >= DV) continue;   // uniform over the 16 lanes of a row
        float pk = 0.f, pq = 0.f;
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            pk += s[p][i].x * kr[4 * i] + s[p][i].y * kr[4 * i + 1] +
                  s[p][i].z * kr[4 * i + 2] + s[p][i].w * kr[4 * i + 3];
            pq += s[p][i].x * qr[4 * i] + s[p][i].y * qr[4 * i + 1] +
                  s[p][i].z * qr[4 * i + 2] + s[p][i].w * qr[4 * i + 3];
        }
        pk = sum16(pk);
        pq = sum16(pq);
        const float vr = to_f32(v[(size_t)unit * DV + row[p]]);
        const float u = b * (vr - a * pk);
        float4 *sp = reinterpret_cast<float4 *>(S + ((size_t)unit * DV + row[p]) * DK + c * VEC);
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            float4 n;
            n.x = a * s[p][i].x + u * kr[4 * i];
            n.y = a * s[p][i].y + u * kr[4 * i + 1];
            n.z = a * s[p][i].z + u * kr[4 * i + 2];
            n.w = a * s[p][i].w + u * kr[4 * i + 3];
            sp[i] = n;
        }
        if (c == 0) o[(size_t)unit * DV + row[p]] = from_f32<TO>(a * pq + u * kq);
    }
}

template <int DK, typename TI, typename TO>
hipError_t launch_step_t(int B, int H, int DV, const void *q, const void *k,
                         const void *v, const float *la, const float *beta,
                         float *S, void *o, hipStream_t st) {
    dim3 grid(B * H, (DV + kStepRowsPerWG - 1) / kStepRowsPerWG);
    hipLaunchKernelGGL((step_kernel<DK, TI, TO>), grid, dim3(256), 0, st, DV,
                       (const TI *)q, (const TI *)k, (const TI *)v, la, beta, S,
                       (TO *)o);
    return hipGetLastError();
}

// io_bf16 / o_bf16 select bfloat16 (else fp32) for q,k,v and for o.
hipError_t launch_step(int B, int H, int DK, int DV, bool io_bf16, bool o_bf16,
                       const void *q, const void *k, const void *v,
                       const float *la, const float *beta, float *S, void *o,
                       hipStream_t st) {
#define GDN_STEP_CASE(DKV, TI, TO)                                                 \
    return launch_step_t<DKV, TI, TO>(B, H, DV, q, k, v, la, beta, S, o, st)
    if (DK == 128) {
        if (io_bf16) { if (o_bf16) GDN_STEP_CASE(128, bf16, bf16); GDN_STEP_CASE(128, bf16, float); }
        if (o_bf16) GDN_STEP_CASE(128, float, bf16);
        GDN_STEP_CASE(128, float, float);
    }
    if (DK == 64) {
        if (io_bf16) { if (o_bf16) GDN_STEP_CASE(64, bf16, bf16); GDN_STEP_CASE(64, bf16, float); }
        if (o_bf16) GDN_STEP_CASE(64, float, bf16);
        GDN_STEP_CASE(64, float, float);
    }
#undef GDN_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
