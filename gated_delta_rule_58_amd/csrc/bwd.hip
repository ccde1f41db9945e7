// Backward pass of the chunkwise gated delta rule on gfx950 (fp32-accurate MFMA).
//
// The pages name a gate-aware backward pass for the chunkwise algorithm
// ("Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention",
// abstract) but print none; this is the chain rule taken through the WY/UT
// chunk steps (research-map summary of "Gated Delta Networks: Improving
// Mamba2 with Delta Rule", section "Approach"; blog "Gated DeltaNet:
// Harmonizing Gating and the Delta Rule for Superior Linear RNNs", section
// "Hardware-Efficient Training").  Per chunk of n <= 64 tokens, with S the
// state entering it, dS' the gradient of the state leaving it, g the
// chunk-local prefix of log alpha, G[r,i] = e^{g_r - g_i} (i <= r),
// A = strict(beta G o K K^T), T = (I + A)^{-1}, P = tril(Q K^T) o G:
//
//   Delta  = T diag(beta) (V - diag(e^g) K S^T)            (forward values)
//   dDelta = P^T dO + diag(e^{g_n - g}) K dS'^T
//   dS     = e^{g_n} dS' + dO^T diag(e^g) Q - F^T K,  F = diag(beta e^g) T^T dDelta
//
// so the state gradients run over the chunks in reverse, and each chunk's
// gradients need only (S, dS'):
//
//   dP = tril(dO Delta^T), dQK = dP o G, dW = -dDelta S
//   dQ = diag(e^g) dO S + dQK K
//   dV = diag(beta) T^T dDelta
//   dT = dDelta (beta V)^T + dW (beta e^g K)^T,  dA = -strict(T^T dT T^T)
//   dK = dQK^T Q + diag(e^{g_n - g}) Delta dS' + diag(beta e^g) T^T dW
//        + dG K + dG^T K,  dG = dA o beta_r G
//   dbeta, dg: row sums of the same products; dlog_alpha = reverse
//   cumulative sum of dg within the chunk.
//
// Five launches.  Every product is fp32-accurate: most run on
// v_mfma_f32_16x16x4_f32 (inputs are exact in fp32); with bf16 inputs, the
// products that have a bf16 input (K, Q, V) as one operand run on the
// 16x16x32 bf16 MFMA, exact when both operands are inputs and otherwise over
// three bf16 pieces that add up to the fp32 operand exactly (split3); the
// sprod products split both fp32 operands so and sum six piece products:
//   1. prep     (one workgroup per chunk and head): T and P;
//   2. states   (one per sequence, head and 64-column d_v slice, chunks in
//               order): the state entering every chunk and Delta (bf16
//               inputs: loader waves copy the next chunk into LDS while
//               consumer waves run the current one);
//   3. dstates  (same grid, chunks in reverse): dS' of every chunk, dDelta,
//               and dS0 (bf16 inputs: split by role like states);
//   4. sprod    (per chunk and head): dO S, -dDelta S, Delta dS', <dS', S>;
//   5. grads    (per chunk and head): dq, dk, dv, dlog_alpha, dbeta.
// Intermediates go through the caller's workspace (layout in bwd_ws_bytes).
//
// fp32 MFMA layout (v_mfma_f32_16x16x4_f32): lane l supplies A[l & 15][l >> 4]
// and B[l >> 4][l & 15] and holds D[4 (l >> 4) + j][l & 15], j = 0..3.
#include "fp32_tiles.h"
#include "img_tiles.h"

namespace gdn {
namespace {

using namespace tiles;
using namespace img;

// ---------------------------------------------------------------- 1. prep
template <int D, typename TI>
__global__ __launch_bounds__(512) void bwd_prep_kernel(
    int T, int H, int units, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ q, const TI *__restrict__ k, const float *__restrict__ la,
    const float *__restrict__ beta, float *__restrict__ wsT, float *__restrict__ wsP, int nch) {
    constexpr int LI = ldx<TI, D>();
    __shared__ __attribute__((aligned(16))) TI sK[BC * LI];
    __shared__ __attribute__((aligned(16))) TI sQ[BC * LI];
    __shared__ __attribute__((aligned(16))) float sA[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sX[BC * LDN];
    __shared__ float sg[4][BC];
    const int tid = threadIdx.x, wave = tid >> 6;
    // Persistent over the (chunk slot, head) pairs ci = blockIdx.x + j gridDim.x:
    // the next pair's K, Q rows and gates load into registers while this one
    // is computed (rows past a ragged end are zero).
    Prefetch<D, TI> pk, pq;
    float gx = 0.f, gb = 0.f;
    auto next = [&](int c) {   // first pair >= c with a chunk (unused slots skipped), and fetch it
        long r0;
        int nv;
        for (; c < nch; c += gridDim.x) {
            if (!slot_chunk(c / H, units, T, NC, varlen, cu, r0, nv)) continue;
            const size_t g0 = (size_t)r0 * H * D + (size_t)(c % H) * D;
            pk.fetch(k + g0, (size_t)H * D, nv, tid);
            pq.fetch(q + g0, (size_t)H * D, nv, tid);
            if (wave == 0) gate_fetch(la, beta, r0, nv, H, c % H, tid & 63, gx, gb);
            break;
        }
        return c;
    };
    for (int ci = next(blockIdx.x); ci < nch;) {
    // the lane index passes through an empty asm statement each iteration, so
    // per-lane addresses are recomputed rather than kept live across the loop
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    const size_t ch = ci;
    pk.commit(sK, LI, tid);
    pq.commit(sQ, LI, tid);
    zero_upper(sX, tid);   // the inverse writes the rest of T
    if (wave == 0) gate_scan(sg, gx, gb, lane);
    __syncthreads();
    const int cn = next(ci + (int)gridDim.x);
    // waves 0-3: rows 16w.. of K K^T -> A; waves 4-7: the same rows of Q K^T -> P
    {
        const int tr = wave & 3;
        const bool isP = wave >= 4;
        const TI *Ar = (isP ? sQ : sK) + 16 * tr * LI;
        float *P = wsP + ch * BC * BC;
        f32x4 g4[4];   // all 4 tiles (upper ones unused)
        zero_n(g4);
        if constexpr (sizeof(TI) == 2) {
            // bf16 inputs: the products are exact in fp32, so the 16x16x32
            // bf16 MFMA (fp32 accumulation) computes the same sums as fp32
            // MFMA; row fragments of 8 consecutive k per lane group
            const int li = lane & 15, lq = lane >> 4;
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Ar + li * LI + 32 * ks + 8 * lq);
#pragma unroll
                for (int tj = 0; tj < 4; ++tj)
                    g4[tj] = mfma32(a, *reinterpret_cast<const bf16x8 *>(sK + (16 * tj + li) * LI + 32 * ks + 8 * lq), g4[tj]);
            }
        } else {
            mmn<D, 4>(Ar, LI, 1, sK, 1, LI, 16 * LI, g4, lane);
        }
        for (int tj = 0; tj < 4; ++tj) {
            const f32x4 acc = g4[tj];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * tr + 4 * (lane >> 4) + j, i = 16 * tj + (lane & 15);
                const float dec = i <= r ? __expf(sg[0][r] - sg[0][i]) : 0.f;
                if (isP) P[r * BC + i] = dec * acc[j];
                else sA[r * LDN + i] = i < r ? sg[2][r] * dec * acc[j] : 0.f;
            }
        }
    }
    __syncthreads();
    block_inverse64(sA, sX, wave, lane);
    {
        float *Tm = wsT + ch * BC * BC;
        for (int e = tid; e < BC * BC / 4; e += 512)
            *reinterpret_cast<f32x4 *>(Tm + 4 * e) =
                *reinterpret_cast<const f32x4 *>(sX + (e >> 4) * LDN + (e & 15) * 4);
    }
    __syncthreads();   // the next pair overwrites every LDS buffer
    ci = cn;
    }
}

// ---------------------------------------------------------------- 2. states
template <int D, typename TI>
__global__ __launch_bounds__(512) void bwd_states_kernel(
    int T, int H, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ k, const TI *__restrict__ v, const float *__restrict__ la,
    const float *__restrict__ beta, const float *__restrict__ S0, const float *__restrict__ wsT,
    float *__restrict__ wsH, float *__restrict__ wsDl) {
    constexpr int LI = ldx<TI, D>(), LF = D + 4, NTC = D / 32, NSL = D / 64;
    __shared__ __attribute__((aligned(16))) TI sK[BC * LI];
    __shared__ __attribute__((aligned(16))) float sS[BC * LF];   // state slice: d_v rows x d_k
    __shared__ __attribute__((aligned(16))) float sT[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sZ[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sD[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sV[BC * LDN];  // V slice
    __shared__ float sg[4][BC];
    const int uh = blockIdx.x / NSL, dv0 = 64 * (blockIdx.x % NSL);
    const int u = uh / H, h = uh % H;
    long start, L;
    unit_span(u, T, varlen, cu, start, L);
    const int N = (int)((L + BC - 1) / BC);
    const int base = unit_base(u, NC, varlen, cu);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int tr = wave & 3, tc0 = (wave >> 2) * NTC;
    f32x4 st[NTC];   // st[t][j] = S[dv0 + 16 tr + 4 lq + j][16 (tc0 + t) + li]
#pragma unroll
    for (int t = 0; t < NTC; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
            st[t][j] = S0 ? S0[((size_t)uh * D + dv0 + row) * D + col] : 0.f;
        }
    Prefetch<D, TI> pk;
    Prefetch<64, TI> pv;
    Prefetch<BC, float> pt;
    float gx = 0.f, gb = 0.f;
    auto fetch = [&](int c) {
        const long row0 = start + (long)c * BC;
        const int n = (int)min((long)BC, L - (long)c * BC);
        const size_t ch = (size_t)(base + c) * H + h;
        pk.fetch(k + ((size_t)row0 * H + h) * D, (size_t)H * D, n, tid);
        pv.fetch(v + ((size_t)row0 * H + h) * D + dv0, (size_t)H * D, n, tid);
        pt.fetch(wsT + ch * BC * BC, BC, BC, tid);
        if (wave == 0) gate_fetch(la, beta, row0, n, H, h, lane, gx, gb);
    };
    if (N > 0) fetch(0);
    for (int c = 0; c < N; ++c) {
        const size_t ch = (size_t)(base + c) * H + h;
        const int n = (int)min((long)BC, L - (long)c * BC);
        float *Hm = wsH + ch * D * D;
#pragma unroll
        for (int t = 0; t < NTC; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
                sS[row * LF + col] = st[t][j];
            }
        pk.commit(sK, LI, tid);
        pv.commit(sV, LDN, tid);
        pt.commit(sT, LDN, tid);
        if (wave == 0) gate_scan(sg, gx, gb, lane);
        __syncthreads();
        if (c + 1 < N) fetch(c + 1);   // next chunk's operands load during this one
        for (int e = tid; e < BC * D / 4; e += 512) {   // the state entering chunk c
            const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
            *reinterpret_cast<f32x4 *>(Hm + (size_t)(dv0 + row) * D + c4) =
                *reinterpret_cast<const f32x4 *>(sS + row * LF + c4);
        }
        // Z = diag(beta) (V - diag(e^g) K S^T), 64 tokens x 64 slice columns
        {
            const int ty = tr, tx0 = 2 * (wave >> 2);
            f32x4 y[2];
            zero_n(y);
            mmn<D, 2>(sK + 16 * ty * LI, LI, 1, sS + 16 * tx0 * LF, 1, LF, 16 * LF, y, lane);
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * ty + 4 * lq + j, col = 16 * (tx0 + x) + li;
                    sZ[r * LDN + col] = sg[2][r] * (sV[r * LDN + col] - sg[1][r] * y[x][j]);
                }
        }
        __syncthreads();
        // Delta = T Z; the state update uses diag(e^{g_n - g}) Delta
        {
            const int ty = tr, tx0 = 2 * (wave >> 2);
            f32x4 d[2];
            zero_n(d);
            mmn<BC, 2>(sT + 16 * ty * LDN, LDN, 1, sZ + 16 * tx0, LDN, 1, 16, d, lane);
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * ty + 4 * lq + j, col = 16 * (tx0 + x) + li;
                    sD[r * LDN + col] = d[x][j] * sg[3][r];
                    if (r < n) wsDl[(ch * BC + r) * D + dv0 + col] = d[x][j];
                }
        }
        __syncthreads();
        // S <- e^{g_n} S + (diag(e^{g_n - g}) Delta)^T K
        const float egn = sg[1][BC - 1];
#pragma unroll
        for (int t = 0; t < NTC; ++t) st[t] = st[t] * egn;
        mmn<BC, NTC>(sD + 16 * tr, 1, LDN, sK + 16 * tc0, LI, 1, 16, st, lane);
        __syncthreads();
    }
}

// The same launch for bf16 inputs.  K S^T and the state update have a bf16
// operand (K), whose products with bf16 values are exact in fp32; the fp32
// operand (S, Delta~) is written as three bf16 pieces hi + mid + lo that add
// up to it exactly (split3), so 16x16x32 bf16 MFMAs over the three pieces
// give the fp32 sums at 3 bf16 MFMAs per 8 fp32 ones.  T Z stays fp32.
__device__ __forceinline__ void split3(float x, bf16 &h, bf16 &m, bf16 &l) {
    h = (bf16)x;
    const float r = x - (float)h;
    m = (bf16)r;
    l = (bf16)(r - (float)m);
}

// Two D tiles (rows 0-15 and 16-31 of a 32-row block) as a D-order operand
// in three bf16 pieces that add up to it exactly.
__device__ __forceinline__ void split3_op(f32x4 d0, f32x4 d1, bf16x8 (&p)[3]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bf16 h, m, l;
        split3(e < 4 ? d0[e] : d1[e - 4], h, m, l);
        p[0][e] = h;
        p[1][e] = m;
        p[2][e] = l;
    }
}

// The six piece products of X Y that reach 2^-16 of the leading one (the
// three left out are below 2^-23 of it).
__device__ __forceinline__ f32x4 mfma_x6(const bf16x8 (&x)[3], const bf16x8 (&y)[3], f32x4 acc) {
    acc = mfma32(x[0], y[0], acc);
    acc = mfma32(x[0], y[1], acc);
    acc = mfma32(x[1], y[0], acc);
    acc = mfma32(x[0], y[2], acc);
    acc = mfma32(x[1], y[1], acc);
    acc = mfma32(x[2], y[0], acc);
    return acc;
}

// The states launch with bf16 inputs: one workgroup per (sequence, head,
// 64 columns of d_v), chunks in order, two phases per chunk:
//   A. store the state entering the chunk; Y = K S^T (S^T in its three
//      exact pieces against exact bf16 K); Z = diag(beta)(V - diag(e^g) Y);
//      Delta = T Z over the six piece products of T and Z; store Delta;
//   B. S <- e^{g_n} S + (diag(e^{g_n - g}) Delta)^T K (exact pieces of
//      Delta~ against K, read transposed).
// Waves 0-3 load the next chunk meanwhile: K, the V slice and T by direct
// global-to-LDS copies into the other of two buffers (K rows XOR-swizzled by
// 16-byte piece through the copy's source addresses, so fragment reads of
// 16 rows hit distinct banks), the gates by a scan in wave 0, and in phase B
// each wave splits the rows of T it copied into T's three exact pieces.
// Waves 4-7 own 16 columns of d_v each, S^T (d_k x 16, fp32) in
// accumulator tiles.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_states_pipe_kernel(
    int T, int H, int NC, int varlen, int xcd_map, const int32_t *__restrict__ cu,
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, const float *__restrict__ la,
    const float *__restrict__ beta, const float *__restrict__ S0, const float *__restrict__ wsT,
    float *__restrict__ wsH, float *__restrict__ wsDl) {
    constexpr int NSL = D / 64, NKS = D / 32, NCT = D / 16;
    constexpr int LC = BC + 8;                 // row stride of T's pieces
    constexpr int KP = D / 8;                  // 16-byte pieces per K row
    constexpr int KROWS = 64 / KP;             // K rows per KB
    constexpr int NKI = BC / KROWS / 4, NVI = BC / 8 / 4, NTI = BC * BC * 4 / 1024 / 4;
    static_assert(NKI * KROWS * 4 == BC && NTI * 4 * 1024 == BC * BC * 4, "copy split");
    __shared__ __attribute__((aligned(16))) bf16 sK[2][BC * D];     // K rows, swizzled
    __shared__ __attribute__((aligned(16))) bf16 sV[2][BC * 64];    // V slice rows
    __shared__ __attribute__((aligned(16))) float sTf[2][BC * BC];  // T as copied
    __shared__ __attribute__((aligned(16))) bf16 sT3[3][BC * LC];   // T's pieces, D-order rows
    __shared__ __attribute__((aligned(16))) float sg[2][4][BC];     // g, e^g, beta, e^{g_n - g}
    // element (r, c) of a K buffer: 16-byte piece c / 8 stored at piece (c / 8) ^ (r % KP)
    auto kidx = [](int r, int c) { return r * D + 8 * ((c >> 3) ^ (r & (KP - 1))) + (c & 7); };

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

    if (wave < 4) {
        // ---- loaders
        auto loader_barrier = [&]() {   // copies are waited for by count beforehand
            __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes done
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // rows past the chunk repeat its last token (beta is 0 there)
        auto copy_chunk = [&](int c, int buf) {
            const long row0 = start + (long)c * BC;
            const int n = (int)min((long)BC, L - (long)c * BC);
            const size_t ch = (size_t)(base + c) * H + h;
#pragma unroll
            for (int s = 0; s < NKI; ++s) {
                const int i = wave + 4 * s, r = KROWS * i + lane / KP, pl = lane % KP;
                lds_dma16(sK[buf] + 512 * i,
                          k + ((size_t)(row0 + min(r, n - 1)) * H + h) * D + 8 * (pl ^ (r & (KP - 1))));
            }
#pragma unroll
            for (int s = 0; s < NVI; ++s) {
                const int i = wave + 4 * s, r = 8 * i + lane / 8;
                lds_dma16(sV[buf] + 512 * i,
                          v + ((size_t)(row0 + min(r, n - 1)) * H + h) * D + dv0 + 8 * (lane % 8));
            }
#pragma unroll
            for (int s = 0; s < NTI; ++s) {
                const int i = wave + 4 * s;
                lds_dma16(sTf[buf] + 256 * i, wsT + ch * BC * BC + 256 * i + 4 * lane);
            }
        };
        // T's pieces from the rows this wave copied: KB piece i = wave + 4 s holds
        // rows 4 i .. 4 i + 3, 32 D-order groups of 8; the wave's 32 NTI groups
        // are spread over its 64 lanes
        static_assert(NTI * 32 % 64 == 0, "whole groups per lane");
        auto split_t = [&](int buf) {
#pragma unroll
            for (int hh = 0; hh < NTI * 32 / 64; ++hh) {
                const int gi = lane + 64 * hh, s = gi / 32, loc = gi % 32;
                const int r = 4 * (wave + 4 * s) + loc / 8, p = 8 * (loc % 8);
                const int i0 = (p & ~31) + (p & 31) / 2;
                const f32x4 x0 = *reinterpret_cast<const f32x4 *>(sTf[buf] + r * BC + i0);
                const f32x4 x1 = *reinterpret_cast<const f32x4 *>(sTf[buf] + r * BC + i0 + 16);
                bf16x8 pc[3];
                split3_op(x0, x1, pc);
#pragma unroll
                for (int q = 0; q < 3; ++q) *reinterpret_cast<bf16x8 *>(sT3[q] + r * LC + p) = pc[q];
            }
        };
        auto gates = [&](int c, int buf) {   // wave 0, after its gate loads have landed
            float x, bt;
            const long row0 = start + (long)c * BC;
            const int n = (int)min((long)BC, L - (long)c * BC);
            gate_fetch(la, beta, row0, n, H, h, lane, x, bt);
            return f32x4{x, bt, 0.f, 0.f};
        };
        if (N > 0) {
            f32x4 gx = wave == 0 ? gates(0, 0) : zero4();
            copy_chunk(0, 0);
            wait_vm<0>();
            if (wave == 0) gate_scan(sg[0], gx[0], gx[1], lane);
            split_t(0);
        }
        loader_barrier();
        for (int c = 0; c < N; ++c) {
            const int nb = (c + 1) & 1;
            if (c + 1 < N) {   // phase A: the next chunk's copies and gates
                f32x4 gx = zero4();
                if (wave == 0) gx = gates(c + 1, nb);
                copy_chunk(c + 1, nb);
                if (wave == 0) {
                    wait_vm<NKI + NVI + NTI>();
                    gate_scan(sg[nb], gx[0], gx[1], lane);
                }
            }
            loader_barrier();
            if (c + 1 < N) {   // phase B: T's pieces of the next chunk
                wait_vm<0>();
                split_t(nb);
            }
            loader_barrier();
        }
        return;
    }

    // ---- consumers: d_v columns dv0 + 16 cw + li
    const int cw = wave - 4;
    const int vcol = dv0 + 16 * cw + li;
    f32x4 st[NCT];   // st[t][j] = S^T[16 t + 4 lq + j][vcol] = S[vcol][16 t + 4 lq + j]
#pragma unroll
    for (int t = 0; t < NCT; ++t)
        st[t] = S0 ? *reinterpret_cast<const f32x4 *>(S0 + ((size_t)uh * D + vcol) * D + 16 * t + 4 * lq)
                   : zero4();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int c = 0; c < N; ++c) {
        const int cb = c & 1;
        const size_t ch = (size_t)(base + c) * H + h;
        const int n = (int)min((long)BC, L - (long)c * BC);
        const bf16 *K = sK[cb];
        const float(*g)[BC] = sg[cb];
        // ---- phase A
        bf16x8 dp[2][3];   // Delta~ = diag(e^{g_n - g}) Delta: exact pieces, D-order over tokens
        {
            float *Hm = wsH + ch * D * D + (size_t)vcol * D;
#pragma unroll
            for (int t = 0; t < NCT; ++t) *reinterpret_cast<f32x4 *>(Hm + 16 * t + 4 * lq) = st[t];
            f32x4 y[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) y[rt] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bf16x8 sp[3];
                split3_op(st[2 * ks], st[2 * ks + 1], sp);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int r = 16 * rt + li;
                    const bf16x8 a = cat(*reinterpret_cast<const bf16x4 *>(K + kidx(r, 32 * ks + 4 * lq)),
                                         *reinterpret_cast<const bf16x4 *>(K + kidx(r, 32 * ks + 16 + 4 * lq)));
#pragma unroll
                    for (int q = 0; q < 3; ++q) y[rt] = mfma32(a, sp[q], y[rt]);
                }
            }
            f32x4 z[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const bf16x4 vx = lds_read_tr(sV[cb] + (16 * rt + 4 * lq + (li >> 2)) * 64 + 16 * cw + 4 * (li & 3));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    z[rt][j] = g[2][r] * ((float)vx[j] - g[1][r] * y[rt][j]);
                }
            }
            bf16x8 zp[2][3];
            split3_op(z[0], z[1], zp[0]);
            split3_op(z[2], z[3], zp[1]);
            f32x4 dd[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int off = (16 * rt + li) * LC + 32 * ks + 8 * lq;
                    const bf16x8 tp[3] = {ld8(sT3[0] + off), ld8(sT3[1] + off), ld8(sT3[2] + off)};
                    acc = mfma_x6(tp, zp[ks], acc);
                }
                dd[rt] = acc;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    if (r < n) wsDl[(ch * BC + r) * D + vcol] = acc[j];
                    dd[rt][j] = acc[j] * g[3][r];
                }
            }
            split3_op(dd[0], dd[1], dp[0]);
            split3_op(dd[2], dd[3], dp[1]);
        }
        __syncthreads();
        // ---- phase B: S^T <- e^{g_n} S^T + K^T Delta~
        {
            const float egn = g[1][BC - 1];
#pragma unroll
            for (int t = 0; t < NCT; ++t) {
                f32x4 acc = st[t] * egn;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    // K^T rows 16 t + li, tokens 32 ks + 4 lq + j (+ 16): column gathers
                    const int r = 32 * ks + 4 * lq + (li >> 2), cc = 16 * t + 4 * (li & 3);
                    const bf16x8 a = cat(lds_read_tr(K + kidx(r, cc)), lds_read_tr(K + kidx(r + 16, cc)));
#pragma unroll
                    for (int q = 0; q < 3; ++q) acc = mfma32(a, dp[ks][q], acc);
                }
                st[t] = acc;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- 3. dstates
template <int D, typename TI, typename TG>
__global__ __launch_bounds__(512) void bwd_dstates_kernel(
    int T, int H, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ q, const TI *__restrict__ k, const TG *__restrict__ dO,
    const float *__restrict__ la, const float *__restrict__ beta, const float *__restrict__ dST,
    const float *__restrict__ wsT, const float *__restrict__ wsP, float *__restrict__ wsDH,
    float *__restrict__ wsE, float *__restrict__ dS0) {
    constexpr int LI = ldx<TI, D>(), LF = D + 4, NTC = D / 32, NSL = D / 64;
    __shared__ __attribute__((aligned(16))) TI sK[BC * LI];
    __shared__ __attribute__((aligned(16))) TI sQ[BC * LI];
    __shared__ __attribute__((aligned(16))) float sG[BC * LF];   // dS' slice: d_v rows x d_k
    __shared__ __attribute__((aligned(16))) float sP[BC * LDN];  // P, then F
    __shared__ __attribute__((aligned(16))) float sT[BC * LDN];
    __shared__ __attribute__((aligned(16))) float sO[BC * LDN];  // dO slice, then e^g dO
    __shared__ __attribute__((aligned(16))) float sE[BC * LDN];
    __shared__ float sg[4][BC];
    const int uh = blockIdx.x / NSL, dv0 = 64 * (blockIdx.x % NSL);
    const int u = uh / H, h = uh % H;
    long start, L;
    unit_span(u, T, varlen, cu, start, L);
    const int N = (int)((L + BC - 1) / BC);
    const int base = unit_base(u, NC, varlen, cu);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int tr = wave & 3, tc0 = (wave >> 2) * NTC;
    f32x4 st[NTC];   // st[t][j] = dS'[dv0 + 16 tr + 4 lq + j][16 (tc0 + t) + li]
#pragma unroll
    for (int t = 0; t < NTC; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
            st[t][j] = dST ? dST[((size_t)uh * D + dv0 + row) * D + col] : 0.f;
        }
    Prefetch<D, TI> pk, pq;
    Prefetch<64, TG> po;
    Prefetch<BC, float> pp, pt;
    float gx = 0.f, gb = 0.f;
    auto fetch = [&](int c) {
        const long row0 = start + (long)c * BC;
        const int n = (int)min((long)BC, L - (long)c * BC);
        const size_t ch = (size_t)(base + c) * H + h;
        pk.fetch(k + ((size_t)row0 * H + h) * D, (size_t)H * D, n, tid);
        pq.fetch(q + ((size_t)row0 * H + h) * D, (size_t)H * D, n, tid);
        po.fetch(dO + ((size_t)row0 * H + h) * D + dv0, (size_t)H * D, n, tid);
        pp.fetch(wsP + ch * BC * BC, BC, BC, tid);
        pt.fetch(wsT + ch * BC * BC, BC, BC, tid);
        if (wave == 0) gate_fetch(la, beta, row0, n, H, h, lane, gx, gb);
    };
    if (N > 0) fetch(N - 1);
    for (int c = N - 1; c >= 0; --c) {
        const size_t ch = (size_t)(base + c) * H + h;
        const int n = (int)min((long)BC, L - (long)c * BC);
        float *DHm = wsDH + ch * D * D;
#pragma unroll
        for (int t = 0; t < NTC; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
                sG[row * LF + col] = st[t][j];
            }
        pk.commit(sK, LI, tid);
        pq.commit(sQ, LI, tid);
        po.commit(sO, LDN, tid);
        pp.commit(sP, LDN, tid);
        pt.commit(sT, LDN, tid);
        if (wave == 0) gate_scan(sg, gx, gb, lane);
        __syncthreads();
        if (c > 0) fetch(c - 1);   // previous chunk's operands load during this one
        for (int e = tid; e < BC * D / 4; e += 512) {   // gradient of the state leaving chunk c
            const int row = e / (D / 4), c4 = (e % (D / 4)) * 4;
            *reinterpret_cast<f32x4 *>(DHm + (size_t)(dv0 + row) * D + c4) =
                *reinterpret_cast<const f32x4 *>(sG + row * LF + c4);
        }
        // dDelta = P^T dO + diag(e^{g_n - g}) K dS'^T
        {
            const int ty = tr, tx0 = 2 * (wave >> 2);
            f32x4 e1[2], e2[2];
            zero_n(e1);
            zero_n(e2);
            mmn<BC, 2>(sP + 16 * ty, 1, LDN, sO + 16 * tx0, LDN, 1, 16, e1, lane);
            mmn<D, 2>(sK + 16 * ty * LI, LI, 1, sG + 16 * tx0 * LF, 1, LF, 16 * LF, e2, lane);
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * ty + 4 * lq + j, col = 16 * (tx0 + x) + li;
                    const float e = e1[x][j] + sg[3][r] * e2[x][j];
                    sE[r * LDN + col] = e;
                    if (r < n) wsE[(ch * BC + r) * D + dv0 + col] = e;
                }
        }
        __syncthreads();
        // F = diag(beta e^g) T^T dDelta (into sP); dO rows scaled by e^g
        {
            const int ty = tr, tx0 = 2 * (wave >> 2);
            f32x4 f[2];
            zero_n(f);
            mmn<BC, 2>(sT + 16 * ty, 1, LDN, sE + 16 * tx0, LDN, 1, 16, f, lane);
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * ty + 4 * lq + j, col = 16 * (tx0 + x) + li;
                    sP[r * LDN + col] = sg[2][r] * sg[1][r] * f[x][j];
                    sO[r * LDN + col] *= sg[1][r];
                }
        }
        __syncthreads();
        // dS <- e^{g_n} dS' + (e^g dO)^T Q - F^T K
        const float egn = sg[1][BC - 1];
        f32x4 fk[NTC];
#pragma unroll
        for (int t = 0; t < NTC; ++t) st[t] = st[t] * egn;
        zero_n(fk);
        mmn<BC, NTC>(sO + 16 * tr, 1, LDN, sQ + 16 * tc0, LI, 1, 16, st, lane);
        mmn<BC, NTC>(sP + 16 * tr, 1, LDN, sK + 16 * tc0, LI, 1, 16, fk, lane);
#pragma unroll
        for (int t = 0; t < NTC; ++t) st[t] = st[t] - fk[t];
        __syncthreads();
    }
    if (dS0) {
#pragma unroll
        for (int t = 0; t < NTC; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
                dS0[((size_t)uh * D + dv0 + row) * D + col] = st[t][j];
            }
    }
}

// The dstates launch with bf16 inputs, split by role like the states launch:
// one workgroup per (sequence, head, 64 columns of d_v), chunks in reverse,
// two phases per chunk c:
//   1. store dS' (the gradient of the state leaving chunk c); dDelta =
//      P^T dO + diag(e^{g_n - g}) K dS'^T (exact pieces of dS' against
//      exact K; the six piece products of P^T and dO); store dDelta;
//      F = diag(beta e^g) T^T dDelta (six piece products);
//   2. dS <- e^{g_n} dS' - F^T K + (e^g dO)^T Q   (exact pieces of F and of
//      e^g dO against K^T and Q^T).
// Waves 0-3 load meanwhile: in phase 1 Q of chunk c (read in phase 2 only)
// and K (double-buffered), the gates, P and T of chunk c - 1, each wave
// waiting for its own copies before the barrier; in phase 2, when every copy
// is visible, P^T and T^T of chunk c - 1 in their three exact pieces, and dO
// of chunk c - 1.  K and Q rows are XOR-swizzled by 16-byte piece
// through the copies' source addresses.  Waves 4-7 own 16 columns of d_v
// each, dS^T (d_k x 16, fp32) in accumulator tiles.
template <int D, typename TG>
__global__ __launch_bounds__(512, 1) void bwd_dstates_pipe_kernel(
    int T, int H, int NC, int varlen, int xcd_map, const int32_t *__restrict__ cu,
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const TG *__restrict__ dO,
    const float *__restrict__ la, const float *__restrict__ beta, const float *__restrict__ dST,
    const float *__restrict__ wsT, const float *__restrict__ wsP, float *__restrict__ wsDH,
    float *__restrict__ wsE, float *__restrict__ dS0) {
    constexpr int NSL = D / 64, NKS = D / 32, NCT = D / 16;
    constexpr int LC = BC + 8;                 // row stride of the pieces of P^T and T^T
    constexpr int KP = D / 8;                  // 16-byte pieces per K or Q row
    constexpr int KROWS = 64 / KP;             // K or Q rows per KB
    constexpr int NKI = BC / KROWS / 4;        // KB copies per loader wave: K, Q
    constexpr int OROWS = 1024 / (64 * (int)sizeof(TG));   // dO rows per KB
    constexpr int NOI = BC / OROWS / 4, NPI = BC * BC * 4 / 1024 / 4;
    static_assert(NKI * KROWS * 4 == BC && NOI * OROWS * 4 == BC && NPI * 4096 == BC * BC * 4,
                  "copy split");
    __shared__ __attribute__((aligned(16))) bf16 sK[2][BC * D];     // K rows, swizzled
    __shared__ __attribute__((aligned(16))) bf16 sQ[BC * D];        // Q rows, swizzled
    __shared__ __attribute__((aligned(16))) TG sO[BC * 64];         // dO slice rows
    __shared__ __attribute__((aligned(16))) float sPf[BC * BC];     // P as copied
    __shared__ __attribute__((aligned(16))) float sTf[BC * BC];     // T as copied
    __shared__ __attribute__((aligned(16))) bf16 sPT[3][BC * LC];   // P^T pieces, D-order rows
    __shared__ __attribute__((aligned(16))) bf16 sTT[3][BC * LC];   // T^T pieces, D-order rows
    __shared__ __attribute__((aligned(16))) float sg[2][4][BC];     // g, e^g, beta, e^{g_n - g}
    auto kidx = [](int r, int c) { return r * D + 8 * ((c >> 3) ^ (r & (KP - 1))) + (c & 7); };

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
    auto rows_of = [&](int c, long &row0, int &n) {
        row0 = start + (long)c * BC;
        n = (int)min((long)BC, L - (long)c * BC);
    };

    if (wave < 4) {
        // ---- loaders
        auto loader_barrier = [&]() {   // copies are waited for by count beforehand
            __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes done
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // rows past the chunk repeat its last token; the consumers zero what
        // those rows would add
        auto copy_rows = [&](bf16 *dst, const bf16 *src, int c) {   // K or Q, swizzled
            long row0;
            int n;
            rows_of(c, row0, n);
#pragma unroll
            for (int s = 0; s < NKI; ++s) {
                const int i = wave + 4 * s, r = KROWS * i + lane / KP, pl = lane % KP;
                lds_dma16(dst + 512 * i,
                          src + ((size_t)(row0 + min(r, n - 1)) * H + h) * D + 8 * (pl ^ (r & (KP - 1))));
            }
        };
        auto copy_o = [&](int c) {   // dO slice
            long row0;
            int n;
            rows_of(c, row0, n);
            constexpr int OP = 64 / OROWS;   // 16-byte pieces per dO row
#pragma unroll
            for (int s = 0; s < NOI; ++s) {
                const int i = wave + 4 * s, r = OROWS * i + lane / OP;
                lds_dma16(sO + 1024 / sizeof(TG) * i,
                          dO + ((size_t)(row0 + min(r, n - 1)) * H + h) * D + dv0 +
                              (16 / sizeof(TG)) * (lane % OP));
            }
        };
        auto copy_pt = [&](int c) {   // P and T
            const size_t ch = (size_t)(base + c) * H + h;
#pragma unroll
            for (int s = 0; s < NPI; ++s) {
                const int i = wave + 4 * s;
                lds_dma16(sPf + 256 * i, wsP + ch * BC * BC + 256 * i + 4 * lane);
                lds_dma16(sTf + 256 * i, wsT + ch * BC * BC + 256 * i + 4 * lane);
            }
        };
        // P^T and T^T pieces: row r, D-order group p of columns i0..i0+3,
        // i0+16..i0+19 holds X[i][r] (any wave: every copy is visible)
        auto split_pt = [&]() {
#pragma unroll
            for (int s = 0; s < 2 * BC * 8 / 256; ++s) {
                // consecutive lanes take consecutive rows r: the column reads
                // below are then consecutive words
                const int e = (tid & 255) + 256 * s, mx = e / (BC * 8), loc = e % (BC * 8);
                const int r = loc % BC, p = 8 * (loc / BC), i0 = (p & ~31) + (p & 31) / 2;
                const float *X = mx == 0 ? sPf : sTf;
                f32x4 x0, x1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x0[j] = X[(i0 + j) * BC + r];
                    x1[j] = X[(i0 + 16 + j) * BC + r];
                }
                bf16x8 pc[3];
                split3_op(x0, x1, pc);
#pragma unroll
                for (int qq = 0; qq < 3; ++qq)
                    *reinterpret_cast<bf16x8 *>((mx == 0 ? sPT[qq] : sTT[qq]) + r * LC + p) = pc[qq];
            }
        };
        // wave 0: the gate loads are issued before the copies and waited for
        // (by the compiler, by count) at the scan
        auto gate_load = [&](int c, float &x, float &bt) {
            long row0;
            int n;
            rows_of(c, row0, n);
            gate_fetch(la, beta, row0, n, H, h, lane, x, bt);
        };
        if (N > 0) {
            float x = 0.f, bt = 0.f;
            if (wave == 0) gate_load(N - 1, x, bt);
            copy_rows(sK[(N - 1) & 1], k, N - 1);
            copy_pt(N - 1);
            copy_o(N - 1);
            wait_vm<0>();
            if (wave == 0) gate_scan(sg[(N - 1) & 1], x, bt, lane);
        }
        loader_barrier();
        if (N > 0) split_pt();
        loader_barrier();
        for (int c = N - 1; c >= 0; --c) {
            // phase 1
            float x = 0.f, bt = 0.f;
            if (c > 0 && wave == 0) gate_load(c - 1, x, bt);
            copy_rows(sQ, q, c);
            if (c > 0) {
                copy_rows(sK[(c - 1) & 1], k, c - 1);
                copy_pt(c - 1);
                if (wave == 0) gate_scan(sg[(c - 1) & 1], x, bt, lane);
            }
            wait_vm<0>();   // Q(c), and K, P, T of chunk c - 1
            loader_barrier();
            // phase 2: the pieces of P^T and T^T of chunk c - 1, and its dO
            if (c > 0) {
                split_pt();
                copy_o(c - 1);
            }
            wait_vm<0>();
            loader_barrier();
        }
        return;
    }

    // ---- consumers: d_v columns dv0 + 16 cw + li
    const int cw = wave - 4;
    const int vcol = dv0 + 16 * cw + li;
    f32x4 ut[NCT];   // ut[t][j] = dS^T[16 t + 4 lq + j][vcol] = dS[vcol][16 t + 4 lq + j]
#pragma unroll
    for (int t = 0; t < NCT; ++t)
        ut[t] = dST ? *reinterpret_cast<const f32x4 *>(dST + ((size_t)uh * D + vcol) * D + 16 * t + 4 * lq)
                    : zero4();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __syncthreads();
    for (int c = N - 1; c >= 0; --c) {
        const int cb = c & 1;
        const size_t ch = (size_t)(base + c) * H + h;
        long row0;
        int n;
        rows_of(c, row0, n);
        const bf16 *K = sK[cb];   // Q (single buffer) is read in phase 2 only
        const float(*g)[BC] = sg[cb];
        bf16x8 fp[2][3], ep[2][3];   // pieces of F and of e^g dO, D-order over tokens
        // ---- phase 1
        {
            float *DHm = wsDH + ch * D * D + (size_t)vcol * D;
#pragma unroll
            for (int t = 0; t < NCT; ++t) *reinterpret_cast<f32x4 *>(DHm + 16 * t + 4 * lq) = ut[t];
            f32x4 e2[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) e2[rt] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                bf16x8 up[3];
                split3_op(ut[2 * ks], ut[2 * ks + 1], up);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int r = 16 * rt + li;
                    const bf16x8 a = cat(*reinterpret_cast<const bf16x4 *>(K + kidx(r, 32 * ks + 4 * lq)),
                                         *reinterpret_cast<const bf16x4 *>(K + kidx(r, 32 * ks + 16 + 4 * lq)));
#pragma unroll
                    for (int qq = 0; qq < 3; ++qq) e2[rt] = mfma32(a, up[qq], e2[rt]);
                }
            }
            // dO at tokens 32 ks + 4 lq + j (+ 16) of this column, zero past the chunk
            bf16x8 op[2][3];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                f32x4 o0, o1, s0, s1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r0 = 32 * ks + 4 * lq + j, r1 = r0 + 16;
                    o0[j] = r0 < n ? to_f32(sO[r0 * 64 + 16 * cw + li]) : 0.f;
                    o1[j] = r1 < n ? to_f32(sO[r1 * 64 + 16 * cw + li]) : 0.f;
                    s0[j] = o0[j] * g[1][r0];
                    s1[j] = o1[j] * g[1][r1];
                }
                split3_op(o0, o1, op[ks]);
                split3_op(s0, s1, ep[ks]);
            }
            f32x4 dd[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int off = (16 * rt + li) * LC + 32 * ks + 8 * lq;
                    const bf16x8 xp[3] = {ld8(sPT[0] + off), ld8(sPT[1] + off), ld8(sPT[2] + off)};
                    acc = mfma_x6(xp, op[ks], acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    dd[rt][j] = acc[j] + g[3][r] * e2[rt][j];
                    if (r < n) wsE[(ch * BC + r) * D + vcol] = dd[rt][j];
                }
            }
            bf16x8 dp[2][3];
            split3_op(dd[0], dd[1], dp[0]);
            split3_op(dd[2], dd[3], dp[1]);
            f32x4 f[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int off = (16 * rt + li) * LC + 32 * ks + 8 * lq;
                    const bf16x8 xp[3] = {ld8(sTT[0] + off), ld8(sTT[1] + off), ld8(sTT[2] + off)};
                    acc = mfma_x6(xp, dp[ks], acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    f[rt][j] = g[2][r] * g[1][r] * acc[j];
                }
            }
            split3_op(f[0], f[1], fp[0]);
            split3_op(f[2], f[3], fp[1]);
        }
        __syncthreads();
        // ---- phase 2: dS^T <- e^{g_n} dS'^T - K^T F + Q^T (e^g dO)
        {
            const float egn = g[1][BC - 1];
#pragma unroll
            for (int t = 0; t < NCT; ++t) {
                f32x4 kf = zero4(), qe = ut[t] * egn;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int r = 32 * ks + 4 * lq + (li >> 2), cc = 16 * t + 4 * (li & 3);
                    const bf16x8 a = cat(lds_read_tr(K + kidx(r, cc)), lds_read_tr(K + kidx(r + 16, cc)));
                    const bf16x8 aq = cat(lds_read_tr(sQ + kidx(r, cc)), lds_read_tr(sQ + kidx(r + 16, cc)));
#pragma unroll
                    for (int qq = 0; qq < 3; ++qq) {
                        kf = mfma32(a, fp[ks][qq], kf);
                        qe = mfma32(aq, ep[ks][qq], qe);
                    }
                }
                ut[t] = qe - kf;
            }
        }
        __syncthreads();
    }
    if (dS0) {
#pragma unroll
        for (int t = 0; t < NCT; ++t)
            *reinterpret_cast<f32x4 *>(dS0 + ((size_t)uh * D + vcol) * D + 16 * t + 4 * lq) = ut[t];
    }
}

// ---------------------------------------------------------------- 4. sprod
// X M for 64 x D row blocks X and a D x D fp32 matrix M, both with up to 24
// significant bits: each operand is written as three bf16 pieces that add up
// to it exactly (split3), and the six piece products down to 2^-16 of the
// leading one run on the 16x16x32 bf16 MFMA with fp32 sums; the three left
// out are below 2^-23 of it, under the fp32 rounding of the sums.  (Eight
// fp32 16x16x4 MFMAs of 32 cycles become six bf16 ones of 16.)  M passes
// through LDS 64 rows (k) at a time as its three pieces, row-major with the
// 8-byte chunks of row r permuted by sp_swz(r), and reaches the MFMA by
// column gathers (transpose reads), whose k order within a 32-step is
// 4 lq + j, then 16 + 4 lq + j; the X fragments follow that order.
constexpr int SP_KR = 64;   // rows of M per LDS round
__device__ __forceinline__ int sp_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
template <int W> __device__ __forceinline__ int sp_pos(int r, int c) {   // element (r, c)
    return r * W + 4 * ((c >> 2) ^ sp_swz(r)) + (c & 3);
}
// B operand of output columns 16 cb .. 16 cb + 15 and k step ks of a piece:
// element (i, e) = piece[32 ks + k(e)][16 cb + i].
template <int W>
__device__ __forceinline__ bf16x8 sp_bfrag(const bf16 *piece, int cb, int ks, int lane) {
    const int lm = lane & 15, lg = lane >> 4, j = lm >> 2, q4 = lm & 3;
    const int r = 32 * ks + 4 * lg + j;
    const bf16 *p = piece + r * W + 4 * ((4 * cb + q4) ^ sp_swz(r));
    return cat(lds_read_tr(p), lds_read_tr(p + 16 * W));   // rows r and r + 16 permute alike
}
// A operand of row `row` (zero when !valid), k step ks: elements
// X[row][32 ks + 4 lq + j] and X[row][32 ks + 16 + 4 lq + j], loaded as fp32
// and later split into its three pieces.
template <typename TX>
__device__ __forceinline__ void sp_aload(const TX *rowp, bool valid, int ks, int lq,
                                         f32x4 (&x)[2]) {
    x[0] = zero4();
    x[1] = zero4();
    if (valid) {
        x[0] = ld4f(rowp + 32 * ks + 4 * lq);
        x[1] = ld4f(rowp + 32 * ks + 16 + 4 * lq);
    }
}
__device__ __forceinline__ void sp_asplit(const f32x4 (&x)[2], bf16x8 (&a)[3]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bf16 h, m, l;
        split3(e < 4 ? x[0][e] : x[1][e - 4], h, m, l);
        a[0][e] = h;
        a[1][e] = m;
        a[2][e] = l;
    }
}
// acc += A B over one k step, six piece products (leading terms first).
__device__ __forceinline__ f32x4 sp_mma6(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x4 acc) {
    acc = mfma32(a[0], b[0], acc);
    acc = mfma32(a[0], b[1], acc);
    acc = mfma32(a[1], b[0], acc);
    acc = mfma32(a[0], b[2], acc);
    acc = mfma32(a[1], b[1], acc);
    acc = mfma32(a[2], b[0], acc);
    return acc;
}

template <int D, typename TG>
__global__ __launch_bounds__(512, 2) void bwd_sprod_kernel(
    int T, int H, int units, int NC, int varlen, const int32_t *__restrict__ cu,
    const TG *__restrict__ dO, const float *__restrict__ wsH, const float *__restrict__ wsDH,
    const float *__restrict__ wsDl, const float *__restrict__ wsE, float *__restrict__ wsOS,
    float *__restrict__ wsW, float *__restrict__ wsKt, float *__restrict__ wsSc) {
    constexpr int NTC = D / 32;                  // 16-column output tiles per wave
    constexpr int NR = D / SP_KR;                // LDS rounds per matrix
    constexpr int PER = SP_KR * D / 4 / 512;     // 4-element groups of a round per thread
    static_assert(PER * 512 * 4 == SP_KR * D, "round split");
    // three pieces of 64 rows of M (48 KB at d = 128): two workgroups per CU
    __shared__ __attribute__((aligned(16))) bf16 sM[3][SP_KR * D];
    __shared__ float sred[8];
    const int slot = blockIdx.x / H, h = blockIdx.x % H;
    long row0;
    int n;
    if (!slot_chunk(slot, units, T, NC, varlen, cu, row0, n)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int tr = wave & 3, tc0 = (wave >> 2) * NTC;
    const size_t ch = blockIdx.x;
    const float *const Sm = wsH + ch * D * D, *const DSm = wsDH + ch * D * D;
    const int arow = 16 * tr + li;
    const bool avalid = arow < n;
    const TG *const dOr = dO + ((size_t)(row0 + (avalid ? arow : 0)) * H + h) * D;
    const float *const dEr = wsE + (ch * BC + arow) * D;
    const float *const dLr = wsDl + (ch * BC + arow) * D;
    // this thread's 4-element groups of a round: row e / (D / 4), columns 4 (e % (D / 4)) + 0..3
    auto grp = [&](int q) { return tid + 512 * q; };
    f32x4 mreg[PER];
    auto fetch = [&](const float *M, int rd) {
#pragma unroll
        for (int q = 0; q < PER; ++q)
            mreg[q] = *reinterpret_cast<const f32x4 *>(M + (size_t)rd * SP_KR * D + 4 * grp(q));
    };
    auto put = [&]() {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int e = grp(q), r = e / (D / 4), c = 4 * (e % (D / 4));
            bf16x4 p0, p1, p2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16 a, b, c3;
                split3(mreg[q][j], a, b, c3);
                p0[j] = a;
                p1[j] = b;
                p2[j] = c3;
            }
            const int at = sp_pos<D>(r, c);
            *reinterpret_cast<bf16x4 *>(&sM[0][at]) = p0;
            *reinterpret_cast<bf16x4 *>(&sM[1][at]) = p1;
            *reinterpret_cast<bf16x4 *>(&sM[2][at]) = p2;
        }
    };

    // dO S and -dDelta S (64 x d_k), then Delta dS' with <dS', S> on the way
    f32x4 a[NTC], b[NTC];
    zero_n(a);
    zero_n(b);
    fetch(Sm, 0);
#pragma unroll 1
    for (int rd = 0; rd < NR; ++rd) {
        put();
        __syncthreads();
        if (rd + 1 < NR) fetch(Sm, rd + 1);
        else fetch(DSm, 0);
        // (X fragments loaded a round ahead would take the registers of two
        // workgroups per CU)
#pragma unroll
        for (int kl = 0; kl < 2; ++kl) {
            f32x4 xr[2];
            bf16x8 xo[3], xe[3];
            sp_aload(dOr, avalid, 2 * rd + kl, lq, xr);
            sp_asplit(xr, xo);
            sp_aload(dEr, avalid, 2 * rd + kl, lq, xr);
            sp_asplit(xr, xe);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const bf16x8 bm[3] = {sp_bfrag<D>(sM[0], tc0 + t, kl, lane),
                                      sp_bfrag<D>(sM[1], tc0 + t, kl, lane),
                                      sp_bfrag<D>(sM[2], tc0 + t, kl, lane)};
                a[t] = sp_mma6(xo, bm, a[t]);
                b[t] = sp_mma6(xe, bm, b[t]);
            }
        }
        __syncthreads();   // sM is rewritten next round
    }
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
        // dO S in the gradient kernel's register layout (lane-blocked, rows
        // past n are zero); -dDelta S row-major
        *reinterpret_cast<f32x4 *>(wsOS + ch * BC * D + 4 * (tid * NTC + t)) = a[t];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
            if (r < n) wsW[(ch * BC + r) * D + col] = -b[t][j];
        }
    }
    zero_n(a);
    float dot = 0.f;
#pragma unroll 1
    for (int rd = 0; rd < NR; ++rd) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {   // <dS', S> over this thread's groups
            const f32x4 y = *reinterpret_cast<const f32x4 *>(Sm + (size_t)rd * SP_KR * D + 4 * grp(q));
            dot += mreg[q][0] * y[0] + mreg[q][1] * y[1] + mreg[q][2] * y[2] + mreg[q][3] * y[3];
        }
        put();
        __syncthreads();
        if (rd + 1 < NR) fetch(DSm, rd + 1);
#pragma unroll
        for (int kl = 0; kl < 2; ++kl) {
            f32x4 xr[2];
            bf16x8 xd[3];
            sp_aload(dLr, avalid, 2 * rd + kl, lq, xr);
            sp_asplit(xr, xd);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const bf16x8 bm[3] = {sp_bfrag<D>(sM[0], tc0 + t, kl, lane),
                                      sp_bfrag<D>(sM[1], tc0 + t, kl, lane),
                                      sp_bfrag<D>(sM[2], tc0 + t, kl, lane)};
                a[t] = sp_mma6(xd, bm, a[t]);
            }
        }
        if (rd + 1 < NR) __syncthreads();
    }
#pragma unroll
    for (int t = 0; t < NTC; ++t)   // Delta dS', lane-blocked as dO S
        *reinterpret_cast<f32x4 *>(wsKt + ch * BC * D + 4 * (tid * NTC + t)) = a[t];
    dot = sum16(dot);
    dot = sum_rows(dot);
    if (lane == 0) sred[wave] = dot;
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int w = 0; w < 8; ++w) s += sred[w];
        wsSc[ch] = s;
    }
}

// ---------------------------------------------------------------- 5. grads
// Products of two row-major operands, A B^T, with both read by rows: lane
// (li, lq) of a 16-row tile supplies the W consecutive elements
// row[4 W s + W lq .. + W - 1] for s < K / (4 W), and MFMA step (s, m) takes
// element m of them, so the k order is the same for every operand whatever
// its source (registers loaded straight from global memory, 16 bytes per
// lane, or LDS rows).
// W elements of X per lane and group: 16 bytes of the input tensors' type.
typedef float f32x8 __attribute__((ext_vector_type(8)));
template <typename X, int W> struct RowVec;
template <> struct RowVec<bf16, 4> { typedef bf16x4 type; };
template <> struct RowVec<bf16, 8> { typedef bf16x8 type; };
template <> struct RowVec<float, 4> { typedef f32x4 type; };
template <> struct RowVec<float, 8> { typedef f32x8 type; };
template <typename X> constexpr int row_w() { return sizeof(X) == 2 ? 8 : 4; }

// W fp32 elements of an LDS row (16-byte aligned)
template <int W> __device__ __forceinline__ auto lds_w(const float *p) {
    if constexpr (W == 4) {
        return *reinterpret_cast<const f32x4 *>(p);
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
}
// Fragments of row r of a chunk of a [tokens, H, D] tensor (zero past n);
// src points at the chunk's row 0, rows are `stride` elements apart.
template <int D, int W, typename X>
__device__ __forceinline__ void row_frags(typename RowVec<X, W>::type (&f)[D / (4 * W)],
                                          const X *src, int stride, int r, int n, int lq) {
    typedef typename RowVec<X, W>::type VT;
    const X *p = src + (r < n ? r : 0) * stride + W * lq;
#pragma unroll
    for (int s = 0; s < D / (4 * W); ++s) {
        f[s] = VT{};
        if (r < n) f[s] = *reinterpret_cast<const VT *>(p + 4 * W * s);
    }
}
// acc[t] += sum_k A(li, k) B_t(li, k) over k < K: fa(s) and fb(t, s) give
// the lane's W elements of group s.
// The operands of group s + 1 are read before the products of group s (they
// stay in their source type until an MFMA takes them), and no instruction
// moves across groups, which bounds the live registers to two groups'
// operands.
template <int K, int W, int NT, typename FA, typename FB>
__device__ __forceinline__ void mm_rows(FA fa, FB fb, f32x4 (&acc)[NT]) {
    constexpr int NS = K / (4 * W);
    auto a = fa(0);
    decltype(fb(0, 0)) b[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) b[t] = fb(t, 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        decltype(a) an = a;
        decltype(fb(0, 0)) bn[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) bn[t] = b[t];
        if (s + 1 < NS) {
            an = fa(s + 1);
#pragma unroll
            for (int t = 0; t < NT; ++t) bn[t] = fb(t, s + 1);
        }
#pragma unroll
        for (int m = 0; m < W; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = mfma_f32(to_f32(a[m]), to_f32(b[t][m]), acc[t]);
        a = an;
#pragma unroll
        for (int t = 0; t < NT; ++t) b[t] = bn[t];
        __builtin_amdgcn_sched_barrier(0);
    }
}

// A B^T with B exact in bf16 (row fragments as above, W = 8) and A fp32
// rows in LDS, split on the fly into three exact bf16 pieces: the fp32 sums
// on 3 bf16 MFMAs per 8 fp32 ones.
__device__ __forceinline__ void split3x8(f32x8 x, bf16x8 &h, bf16x8 &m, bf16x8 &l) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bf16 a, b, c;
        split3(x[e], a, b, c);
        h[e] = a;
        m[e] = b;
        l[e] = c;
    }
}
// acc[t] += A B_t^T, A the fp32 rows at pa (lane offset included), B_t exact
template <int K, int NT>
__device__ __forceinline__ void mm_x3_a(const float *pa, const bf16x8 (&fb)[NT][K / 32],
                                        f32x4 (&acc)[NT]) {
#pragma unroll
    for (int s = 0; s < K / 32; ++s) {
        bf16x8 h, m, l;
        split3x8(lds_w<8>(pa + 32 * s), h, m, l);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            acc[t] = mfma32(h, fb[t][s], acc[t]);
            acc[t] = mfma32(m, fb[t][s], acc[t]);
            acc[t] = mfma32(l, fb[t][s], acc[t]);
        }
    }
}
template <int D, typename TI, typename TG>
__global__ __launch_bounds__(512, 4) void bwd_grads_kernel(
    int T, int H, int units, int NC, int varlen, const int32_t *__restrict__ cu,
    const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
    const TG *__restrict__ dO, const float *__restrict__ la, const float *__restrict__ beta,
    const float *__restrict__ wsT, const float *__restrict__ wsP, const float *__restrict__ wsDl,
    const float *__restrict__ wsE, const float *__restrict__ wsOS, const float *__restrict__ wsW,
    const float *__restrict__ wsKt, const float *__restrict__ wsSc, TG *__restrict__ dq,
    TG *__restrict__ dk, TG *__restrict__ dv, float *__restrict__ dla,
    float *__restrict__ dbeta) {
    constexpr int LI = ldx<TI, D>(), LF = D + 4, NTC = D / 32;
    constexpr int NN = BC * LDN;                                  // a 64 x 64 fp32 block
    constexpr int NB = BC * LF > 2 * NN ? BC * LF : 2 * NN;
    // one group width for every product, so that the summation order (and
    // with it every fp32 result) is the same whichever type dO has
    constexpr int WI = row_w<TI>();
    static_assert(BC * LI * sizeof(TI) <= NN * sizeof(float), "a K or Q tile fits a 64 x 64 block");
    // 73 KB of LDS, so two workgroups share a CU; operands read only by rows
    // (dO, V, K in the first products) come from global memory as fragments.
    //   sN   dQK = dP o G, from the first product to the last
    //   sT   T, then K
    //   sB   Delta, dDelta, dW (64 x d), then dT | M, then dG | Q
    __shared__ __attribute__((aligned(16))) float sN[NN];
    __shared__ __attribute__((aligned(16))) float sT[NN];
    __shared__ __attribute__((aligned(16))) float sB[NB];
    __shared__ float sg[4][BC];
    // per-wave partial row sums of dbeta and dg, added in a fixed order at the
    // end (no atomics: the result does not depend on wave timing)
    __shared__ float sdb[8][BC], sdg[8][BC];
    float *const sB1 = sB + NN;
    TI *const sK = reinterpret_cast<TI *>(sT);
    TI *const sQ = reinterpret_cast<TI *>(sB1);
    const int slot = blockIdx.x / H, h = blockIdx.x % H;
    long row0;
    int n;
    if (!slot_chunk(slot, units, T, NC, varlen, cu, row0, n)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lq = lane >> 4;
    const int tr = wave & 3, tc0 = (wave >> 2) * NTC;   // 64 x D tiles: row tr, columns tc0..
    const int ty = wave & 3, tx0 = 2 * (wave >> 2);     // 64 x 64 tiles: row ty, columns tx0, tx0+1
    const size_t ch = blockIdx.x;
    // chunk origins of the [tokens, H, D] tensors; rows are HD elements apart
    const int HD = H * D;
    const size_t gb = (size_t)row0 * HD + (size_t)h * D;
    const TI *const qc = q + gb, *const kc = k + gb, *const vc = v + gb;
    const TG *const dOc = dO + gb;
    TG *const dqc = dq + gb, *const dkc = dk + gb, *const dvc = dv + gb;
    const float *const Pc = wsP + ch * BC * BC;
#define ADDG(row, x) (sdg[wave][(row)] += (x))
#define ADDB(row, x) (sdb[wave][(row)] += (x))
    for (int e = tid; e < 8 * BC; e += 512) {
        sdb[e / BC][e % BC] = 0.f;
        sdg[e / BC][e % BC] = 0.f;
    }
    typename RowVec<TG, WI>::type fo[D / (4 * WI)];
    row_frags<D, WI>(fo, dOc, HD, 16 * ty + li, n, lq);
    load_ws_rows<D>(sB, LF, wsDl + ch * BC * D, n, tid, 512);   // Delta
    load_nn(sT, wsT + ch * BC * BC, tid, 512);
    Prefetch<D, float> pf;
    pf.fetch(wsE + ch * BC * D, D, n, tid);                     // dDelta, for the next stage
    if (wave == 0) chunk_gates(sg, la, beta, row0, n, H, h, lane);
    __syncthreads();

    // dP = tril(dO Delta^T); dQK = dP o G; dg += rowsum(dP o P) - colsum(dP o P)
    f32x4 a2[2];
    zero_n(a2);
    {
        const float *pb = sB + (16 * tx0 + li) * LF + WI * lq;
        mm_rows<D, WI, 2>([&](int s) { return fo[s]; },
                          [&](int t, int s) { return lds_w<WI>(pb + 16 * t * LF + 4 * WI * s); },
                          a2);
    }
    for (int x = 0; x < 2; ++x) {
        const int tx = tx0 + x;
        const f32x4 a = a2[x];
        float col = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * ty + 4 * lq + j, i = 16 * tx + li;
            const float dp = i <= r ? a[j] : 0.f;
            const float gm = i <= r ? __expf(sg[0][r] - sg[0][i]) : 0.f;
            sN[r * LDN + i] = dp * gm;
            const float m = dp * Pc[r * BC + i];
            const float rs = sum16(m);
            if (li == 0) ADDG(r, rs);
            col += m;
        }
        col = sum_rows(col);
        if (lq == 0) ADDG(16 * tx + li, -col);
    }
    typename RowVec<TI, WI>::type fb[2][D / (4 * WI)];
#pragma unroll
    for (int x = 0; x < 2; ++x) row_frags<D, WI>(fb[x], vc, HD, 16 * (tx0 + x) + li, n, lq);
    __syncthreads();   // Delta no longer read
    pf.commit(sB, LF, tid);
    pf.fetch(wsW + ch * BC * D, D, n, tid);                     // dW, for the next stage
    __syncthreads();

    // dT = dDelta (beta V)^T + ...; dV = diag(beta) T^T dDelta
    f32x4 dt[2];
    zero_n(dt);
    {
        const float *pa = sB + (16 * ty + li) * LF + WI * lq;
        if constexpr (sizeof(TI) == 2)
            mm_x3_a<D, 2>(pa, fb, dt);
        else
            mm_rows<D, WI, 2>([&](int s) { return lds_w<WI>(pa + 4 * WI * s); },
                              [&](int t, int s) { return fb[t][s]; }, dt);
    }
    // T[k][r] at this lane's dT positions (k = 16 ty + 4 lq + j, r = 16 (tx0 + x) + li):
    // a row sum of T^T X o Y is a column sum of T o (X Y^T), and X Y^T is the
    // dT term just formed, so the dbeta and dg row sums below need no
    // elements of V or K
    auto tcolsum = [&](const f32x4 (&w)[2], int x) {
        float cs = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) cs += sT[(16 * ty + 4 * lq + j) * LDN + 16 * (tx0 + x) + li] * w[x][j];
        cs = sum_rows(cs);
        return cs;   // for column r = 16 (tx0 + x) + li, in every lane group
    };
    // dbeta += rows(T^T dDelta . V) = column sums of T o (dDelta V^T)
    for (int x = 0; x < 2; ++x) {
        const float cs = tcolsum(dt, x);
        if (lq == 0) ADDB(16 * (tx0 + x) + li, cs);
    }
    for (int x = 0; x < 2; ++x) dt[x] = dt[x] * sg[2][16 * (tx0 + x) + li];
    f32x4 an[NTC];
    zero_n(an);
    mmn<BC, NTC>(sT + 16 * tr, 1, LDN, sB + 16 * tc0, LF, 1, 16, an, lane);
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
        const int tc = tc0 + t;
        const f32x4 a = an[t];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * tr + 4 * lq + j, col = 16 * tc + li;
            if (r < n) dvc[r * HD + col] = cvt<TG>(sg[2][r] * a[j]);
        }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) row_frags<D, WI>(fb[x], kc, HD, 16 * (tx0 + x) + li, n, lq);
    typename RowVec<TI, WI>::type fk[D / (4 * WI)];
    row_frags<D, WI>(fk, kc, HD, 16 * ty + li, n, lq);
    __syncthreads();   // dDelta no longer read
    pf.commit(sB, LF, tid);
    __syncthreads();

    // dT += dW (beta e^g K)^T; dK = diag(beta e^g) T^T dW + ...; K K^T for dA below
    zero_n(a2);
    f32x4 kk2[2];
    zero_n(kk2);
    {
        const float *pa = sB + (16 * ty + li) * LF + WI * lq;
        if constexpr (sizeof(TI) == 2)
            mm_x3_a<D, 2>(pa, fb, a2);
        else
            mm_rows<D, WI, 2>([&](int s) { return lds_w<WI>(pa + 4 * WI * s); },
                              [&](int t, int s) { return fb[t][s]; }, a2);
        if constexpr (sizeof(TI) == 2) {
            // K K^T of bf16 inputs: exact products, so one 16x16x32 bf16 MFMA
            // per group (the fragments are already in its operand layout)
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t) kk2[t] = mfma32(fk[s], fb[t][s], kk2[t]);
        } else {
            mm_rows<D, WI, 2>([&](int s) { return fk[s]; },
                              [&](int t, int s) { return fb[t][s]; }, kk2);
        }
    }
    // rows(T^T dW . K) = column sums of T o (dW K^T): dbeta += e^g x, dg += beta e^g x
    for (int x = 0; x < 2; ++x) {
        const int i = 16 * (tx0 + x) + li;
        const float cs = tcolsum(a2, x);
        if (lq == 0) {
            ADDB(i, sg[1][i] * cs);
            ADDG(i, sg[2][i] * sg[1][i] * cs);
        }
        dt[x] = dt[x] + a2[x] * (sg[2][i] * sg[1][i]);
    }
    f32x4 dka[NTC];
    zero_n(an);
    mmn<BC, NTC>(sT + 16 * tr, 1, LDN, sB + 16 * tc0, LF, 1, 16, an, lane);
#pragma unroll
    for (int t = 0; t < NTC; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * tr + 4 * lq + j;
            dka[t][j] = sg[2][r] * sg[1][r] * an[t][j];
        }
    __syncthreads();   // dW no longer read
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sB[(16 * ty + 4 * lq + j) * LDN + 16 * (tx0 + x) + li] = dt[x][j];
    __syncthreads();
    // M = T^T dT (into sB1)
    zero_n(a2);
    mmn<BC, 2>(sT + 16 * ty, 1, LDN, sB + 16 * tx0, LDN, 1, 16, a2, lane);
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sB1[(16 * ty + 4 * lq + j) * LDN + 16 * (tx0 + x) + li] = a2[x][j];
    Prefetch<D, TI> pk, pq;
    pk.fetch(kc, HD, n, tid);
    pq.fetch(qc, HD, n, tid);
    __syncthreads();   // M complete; dT no longer read
    // dA = -strict(M T^T); dG = dA o beta_r G (into sB, over dT);
    // dbeta += rowsum(dA o G o K K^T); dg += rowsum(dA o A) - colsum(dA o A)
    zero_n(a2);
    mmn<BC, 2>(sB1 + 16 * ty * LDN, LDN, 1, sT + 16 * tx0 * LDN, 1, LDN, 16 * LDN, a2, lane);
    for (int x = 0; x < 2; ++x) {
        const int tx = tx0 + x;
        const f32x4 a = a2[x], kk = kk2[x];
        float col = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * ty + 4 * lq + j, i = 16 * tx + li;
            const float gm = i < r ? __expf(sg[0][r] - sg[0][i]) : 0.f;
            const float da = i < r ? -a[j] : 0.f;
            const float br = sg[2][r];
            sB[r * LDN + i] = da * br * gm;
            const float t1 = da * gm * kk[j];
            const float rb = sum16(t1);
            const float m = br * t1;   // dA o A
            const float rg = sum16(m);
            if (li == 0) {
                ADDB(r, rb);
                ADDG(r, rg);
            }
            col += m;
        }
        col = sum_rows(col);
        if (lq == 0) ADDG(16 * tx + li, -col);
    }
    // this lane's elements of dO S and Delta dS' (stored lane-blocked by the
    // state-product kernel, whose workgroups tile the chunk the same way)
    f32x4 osv[NTC], ktv[NTC];
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
        osv[t] = *reinterpret_cast<const f32x4 *>(wsOS + ch * BC * D + 4 * (tid * NTC + t));
        ktv[t] = *reinterpret_cast<const f32x4 *>(wsKt + ch * BC * D + 4 * (tid * NTC + t));
    }
    __syncthreads();   // T and M no longer read
    pk.commit(sK, LI, tid);
    pq.commit(sQ, LI, tid);
    __syncthreads();

    // dK = dQK^T Q + diag(e^{g_n - g}) Delta dS' + diag(beta e^g) T^T dW + dG K + dG^T K
    // dg -= s_r, dg_{n-1} += sum_r s_r with s = rows(Delta dS' . K~)
    float ssum = 0.f;
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
        const int tc = tc0 + t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * tr + 4 * lq + j, col = 16 * tc + li;
            const float kt = sg[3][r] * ktv[t][j];
            dka[t][j] += kt;
            const float s = sum16(kt * to_f32(sK[r * LI + col]));
            if (li == 0) ADDG(r, -s);
            ssum += s;   // the same in all 16 lanes of the group
        }
    }
    // dQ = diag(e^g) dO S + dQK K;  dg += e^g rows(dO S . Q)
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
        const int tc = tc0 + t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * tr + 4 * lq + j, col = 16 * tc + li;
            an[t][j] = sg[1][r] * osv[t][j];
            const float rg = sum16(an[t][j] * to_f32(sQ[r * LI + col]));
            if (li == 0) ADDG(r, rg);
        }
    }
    if constexpr (sizeof(TI) == 2) {
        // bf16 inputs: K and Q enter by columns (B fragments of 8 consecutive
        // tokens of one d_k column, exact), dQK and dG by rows or columns as
        // three exact bf16 pieces; one 32-token block at a time
        auto colfrag = [&](const TI *X, int s, int t) {
            bf16x8 f;
#pragma unroll
            for (int m = 0; m < 8; ++m) f[m] = X[(32 * s + 8 * lq + m) * LI + 16 * (tc0 + t) + li];
            return f;
        };
        // rows (unit stride along k) or columns (stride LDN) of a 64 x 64 fp32 block
        auto apieces = [&](const float *X, bool bycol, int s, bf16x8 &h, bf16x8 &m, bf16x8 &l) {
            f32x8 a;
            if (bycol) {
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = X[(32 * s + 8 * lq + e) * LDN + 16 * tr + li];
            } else {
                a = lds_w<8>(X + (16 * tr + li) * LDN + 32 * s + 8 * lq);
            }
            split3x8(a, h, m, l);
        };
        auto acc3 = [&](f32x4 (&acc)[NTC], const bf16x8 &h, const bf16x8 &m, const bf16x8 &l,
                        const bf16x8 (&bf)[NTC]) {
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                acc[t] = mfma32(h, bf[t], acc[t]);
                acc[t] = mfma32(m, bf[t], acc[t]);
                acc[t] = mfma32(l, bf[t], acc[t]);
            }
        };
#pragma unroll
        for (int s = 0; s < BC / 32; ++s) {
            bf16x8 kf[NTC], qf[NTC], h, m, l;
#pragma unroll
            for (int t = 0; t < NTC; ++t) kf[t] = colfrag(sK, s, t);
            apieces(sN, false, s, h, m, l);   // dQK K
            acc3(an, h, m, l, kf);
            apieces(sB, false, s, h, m, l);   // dG K
            acc3(dka, h, m, l, kf);
            apieces(sB, true, s, h, m, l);    // dG^T K
            acc3(dka, h, m, l, kf);
#pragma unroll
            for (int t = 0; t < NTC; ++t) qf[t] = colfrag(sQ, s, t);
            apieces(sN, true, s, h, m, l);    // dQK^T Q
            acc3(dka, h, m, l, qf);
        }
    } else {
        mmn<BC, NTC>(sN + 16 * tr * LDN, LDN, 1, sK + 16 * tc0, LI, 1, 16, an, lane);
        mmn<BC, NTC>(sN + 16 * tr, 1, LDN, sQ + 16 * tc0, LI, 1, 16, dka, lane);
        mmn<BC, NTC>(sB + 16 * tr * LDN, LDN, 1, sK + 16 * tc0, LI, 1, 16, dka, lane);
        mmn<BC, NTC>(sB + 16 * tr, 1, LDN, sK + 16 * tc0, LI, 1, 16, dka, lane);
    }
#pragma unroll
    for (int t = 0; t < NTC; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 16 * tr + 4 * lq + j, col = 16 * (tc0 + t) + li;
            if (r < n) {
                dkc[r * HD + col] = cvt<TG>(dka[t][j]);
                dqc[r * HD + col] = cvt<TG>(an[t][j]);
            }
        }
    ssum = sum_rows(ssum);
    if (lane == 0 && n > 0) ADDG(n - 1, ssum);
#undef ADDG
#undef ADDB
    __syncthreads();
    // dg_{n-1} += e^{g_n} <dS', S>; dlog_alpha = reverse cumulative sum of dg
    if (wave == 0) {
        float x = 0.f, db = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            x += sdg[w][lane];
            db += sdb[w][lane];
        }
        if (lane >= n) x = 0.f;
        if (lane == n - 1) x += sg[1][BC - 1] * wsSc[ch];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(x, off);
            if (lane + off < 64) x += y;
        }
        if (lane < n) {
            const size_t idx = (size_t)(row0 + lane) * H + h;
            dla[idx] = x;
            dbeta[idx] = db;
        }
    }
}

template <int D, typename TI, typename TG>
hipError_t launch_bwd_t(int units, int T, int H, const int32_t *cu, const void *q, const void *k,
                        const void *v, const float *la, const float *beta, const float *S0,
                        const void *dO, const float *dST, void *dq, void *dk, void *dv,
                        float *dla, float *dbeta, float *dS0, float *ws, long nslots,
                        hipStream_t st) {
    const int varlen = cu != nullptr;
    const int NC = varlen ? 0 : (T + BC - 1) / BC;
    const size_t nch = (size_t)nslots * H;
    // Workspace, per chunk slot and head: T and P (64 x 64), the state entering
    // the chunk and the gradient of the state leaving it (d x d), Delta, dDelta,
    // dO S, -dDelta S and Delta dS' (64 x d; dO S and Delta dS' lane-blocked in
    // the gradient kernel's register layout, the others row-major), <dS', S>.
    float *wsT = ws;
    float *wsP = wsT + nch * BC * BC;
    float *wsH = wsP + nch * BC * BC;
    float *wsDH = wsH + nch * D * D;
    float *wsDl = wsDH + nch * D * D;
    float *wsE = wsDl + nch * BC * D;
    float *wsOS = wsE + nch * BC * D;
    float *wsW = wsOS + nch * BC * D;
    float *wsKt = wsW + nch * BC * D;
    float *wsSc = wsKt + nch * BC * D;
    const TI *qi = (const TI *)q, *ki = (const TI *)k, *vi = (const TI *)v;
    const TG *dOg = (const TG *)dO;
    const unsigned seq_grid = (unsigned)((long)units * H * (D / 64));
    const int xcd_map = ((long)units * H) % 8 == 0 ? 1 : 0;   // d_v slices of a head on one XCD
    if (nch > 0)
        // persistent: two workgroups per CU (70 KB of LDS each)
        hipLaunchKernelGGL((bwd_prep_kernel<D, TI>), dim3((unsigned)std::min<size_t>(nch, 512)),
                           dim3(512), 0, st, T, H, units, NC, varlen, cu, qi, ki, la, beta, wsT,
                           wsP, (int)nch);
    if (nch > 0) {
        if constexpr (sizeof(TI) == 2)
            hipLaunchKernelGGL((bwd_states_pipe_kernel<D>), dim3(seq_grid), dim3(512), 0, st, T,
                               H, NC, varlen, xcd_map, cu, ki, vi, la, beta, S0, wsT, wsH, wsDl);
        else
            hipLaunchKernelGGL((bwd_states_kernel<D, TI>), dim3(seq_grid), dim3(512), 0, st, T, H,
                               NC, varlen, cu, ki, vi, la, beta, S0, wsT, wsH, wsDl);
    }
    if constexpr (sizeof(TI) == 2)
        hipLaunchKernelGGL((bwd_dstates_pipe_kernel<D, TG>), dim3(seq_grid), dim3(512), 0, st,
                           T, H, NC, varlen, xcd_map, cu, qi, ki, dOg, la, beta, dST, wsT, wsP,
                           wsDH, wsE, dS0);
    else
        hipLaunchKernelGGL((bwd_dstates_kernel<D, TI, TG>), dim3(seq_grid), dim3(512), 0, st, T,
                           H, NC, varlen, cu, qi, ki, dOg, la, beta, dST, wsT, wsP, wsDH, wsE, dS0);
    if (nch > 0) {
        hipLaunchKernelGGL((bwd_sprod_kernel<D, TG>), dim3((unsigned)nch), dim3(512), 0, st, T, H,
                           units, NC, varlen, cu, dOg, wsH, wsDH, wsDl, wsE, wsOS, wsW, wsKt, wsSc);
        hipLaunchKernelGGL((bwd_grads_kernel<D, TI, TG>), dim3((unsigned)nch), dim3(512), 0, st, T,
                           H, units, NC, varlen, cu, qi, ki, vi, dOg, la, beta, wsT, wsP, wsDl, wsE,
                           wsOS, wsW, wsKt, wsSc, (TG *)dq, (TG *)dk, (TG *)dv, dla, dbeta);
    }
    return hipGetLastError();
}

}  // namespace

bool chunk_bwd_supported(int dk, int dv, int chunk, bool io_bf16) {
    if (chunk != BC || dk != dv) return false;
    return io_bf16 ? (dk == 64 || dk == 128) : dk == 64;
}

// Chunk slots of the workspace: units * ceil(T / 64) for a dense batch,
// floor(T / 64) + n_seqs + 1 for packed sequences.
long chunk_bwd_slots(int units, int T, bool varlen) {
    return varlen ? (long)T / BC + units + 1 : (long)units * ((T + BC - 1) / BC);
}

size_t chunk_bwd_ws_bytes(int units, int T, int H, int d, bool varlen) {
    const size_t nch = (size_t)chunk_bwd_slots(units, T, varlen) * H;
    return sizeof(float) * nch *
           (2 * (size_t)BC * BC + 2 * (size_t)d * d + 5 * (size_t)BC * d + 1);
}

hipError_t launch_chunk_bwd(int units, int T, int H, int d, bool io_bf16, bool g_bf16,
                            const int32_t *cu, const void *q, const void *k, const void *v,
                            const float *la, const float *beta, const float *S0,
                            const void *dO, const float *dST, void *dq, void *dk, void *dv,
                            float *dla, float *dbeta, float *dS0, void *ws, hipStream_t st) {
    const long nslots = chunk_bwd_slots(units, T, cu != nullptr);
    float *w = (float *)ws;
#define GDN_BWD(DV, TI, TG)                                                                   \
    return launch_bwd_t<DV, TI, TG>(units, T, H, cu, q, k, v, la, beta, S0, dO, dST, dq, dk, \
                                    dv, dla, dbeta, dS0, w, nslots, st)
    if (io_bf16) {
        if (d == 128) { if (g_bf16) GDN_BWD(128, bf16, bf16); GDN_BWD(128, bf16, float); }
        if (d == 64) { if (g_bf16) GDN_BWD(64, bf16, bf16); GDN_BWD(64, bf16, float); }
    } else if (d == 64) {
        if (g_bf16) GDN_BWD(64, float, bf16);
        GDN_BWD(64, float, float);
    }
#undef GDN_BWD
    return hipErrorInvalidValue;
}

}  // namespace gdn
