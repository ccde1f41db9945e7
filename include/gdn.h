/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated-delta-rule library, libgdn.so.
 *
 * The operation is the gated delta rule of "Gated Delta Networks: Improving
 * Mamba2 with Delta Rule" (research-map summary, section "Approach"; blog
 * "Gated DeltaNet: Harmonizing Gating and the Delta Rule for Superior Linear
 * RNNs", section "Methodology: The Gated Delta Rule"):
 *
 *     S_t = S_{t-1} ( alpha_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T,
 *     o_t = S_t q_t        (read-out of the post-update state, no scale)
 *
 * with the state S_t a d_v x d_k fp32 matrix per (sequence, head).  The
 * pages print no read-out; the one above is the library's definition.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (HIP device memory of the
 *     current device), contiguous, row-major, owned by the caller.  The
 *     library allocates nothing and keeps no device state beyond its loaded
 *     code objects; it is reentrant across streams.
 *   - The gate is passed as log(alpha) in fp32 (alpha in (0,1] means
 *     log_alpha <= 0); beta is fp32.  Any real beta is accepted.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work: it returns before the GPU has run it,
 *     and faults inside a kernel surface at the caller's next stream sync.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     rejected call has no effect and returns a nonzero gdn_status, with a
 *     message available from gdn_last_error() (thread-local).
 *   - Pointers must be 16-byte aligned (GDN_ERR_ALIGNMENT otherwise).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_dtype {
    GDN_F32 = 0,   /* q, k, v, o in fp32 */
    GDN_BF16 = 1   /* q, k, v, o in bfloat16 (fp32 state and accumulation) */
} gdn_dtype;

/* Optional input prologue, fused into the kernels (bit flags, OR-ed): the
 * step just before the recurrence, which turns raw projections into its
 * inputs.  The pages define no normalisation of q and k and no
 * parametrisation of alpha and beta; the library's definitions are
 *   GDN_PROLOGUE_NORM_QK  q <- q / max(|q|, 1e-6), k <- k / max(|k|, 1e-6)
 *                         per token and head, in fp32 on the loaded values;
 *   GDN_PROLOGUE_GATES    the log_alpha argument carries a pre-activation a
 *                         and beta carries a pre-activation b;
 *                         log alpha = -softplus(a), beta = sigmoid(b).
 * 0 means q, k, log_alpha and beta are used as given. */
typedef enum gdn_prologue {
    GDN_PROLOGUE_NONE = 0,
    GDN_PROLOGUE_NORM_QK = 1,
    GDN_PROLOGUE_GATES = 2
} gdn_prologue;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,  /* null required pointer, negative/zero dims, varlen with B != 1,
                                 unknown prologue bits */
    GDN_ERR_UNSUPPORTED = 2,  /* (d_k, d_v, chunk, dtype) with no compiled kernel, or
                                 H > 32768 (the kernels' 32-bit row offsets) */
    GDN_ERR_ALIGNMENT = 3,    /* a pointer not 16-byte aligned */
    GDN_ERR_WORKSPACE = 4,    /* workspace smaller than gdn_chunk_fwd_workspace_size */
    GDN_ERR_HIP = 5           /* a HIP launch error */
} gdn_status;

/* Problem descriptor of gdn_chunk_fwd.
 *   B, T, H   batch, tokens per batch row, heads (T may be 0);
 *   d_k, d_v  key and value widths;
 *   chunk     chunk length C of the chunkwise algorithm (any value gives the
 *             same result up to rounding; only compiled values are accepted);
 *   n_seqs    0 for a dense batch, else the number of sequences packed into
 *             one row of T tokens (then B must be 1 and cu_seqlens given);
 *   io_dtype  a gdn_dtype for q, k, v;
 *   o_dtype   a gdn_dtype for o.  GDN_F32 is the exact-parity choice: the
 *             read-outs are heavy-tailed (max |o| is 10-20x RMS(o) on
 *             random inputs), so rounding o to bf16 alone moves the largest
 *             outputs by up to ~4% of RMS(o);
 *   prologue  OR of gdn_prologue flags (0: inputs used as given). */
typedef struct gdn_shape {
    int B, T, H, d_k, d_v, chunk;
    int n_seqs;
    int io_dtype;
    int o_dtype;
    int prologue;
} gdn_shape;

/* Bytes of device workspace gdn_chunk_fwd needs for `shape` (written to
 * *bytes).  The current kernels need none (0), but callers should query and
 * pass it so that future kernels can use one.  Returns a gdn_status. */
int gdn_chunk_fwd_workspace_size(const gdn_shape *shape, size_t *bytes);

/* Chunkwise-parallel forward pass of the gated delta rule over whole
 * sequences: the extended WY/UT chunk algorithm (research-map summary,
 * section "Approach"; blog, section "Hardware-Efficient Training"), which
 * reaches the token recurrence's result exactly up to rounding.
 *
 *   q, k        [B, T, H, d_k]  io_dtype
 *   v           [B, T, H, d_v]  io_dtype
 *   log_alpha   [B, T, H]       fp32, log of the gate alpha_t
 *   beta        [B, T, H]       fp32
 *   S0          [U, H, d_v, d_k] fp32 initial states, U = B (dense) or
 *               n_seqs (packed); NULL means zeros.
 *   cu_seqlens  [n_seqs + 1]    int32 device array of sequence offsets
 *               (cu[0] = 0, non-decreasing, cu[n_seqs] = T; precondition,
 *               not checked); NULL for a dense batch.  Empty sequences are
 *               allowed.  The chunk grid restarts at every sequence start
 *               and each sequence starts from its own S0.
 *   o           [B, T, H, d_v]  o_dtype output; must not alias an input.
 *   S_T         [U, H, d_v, d_k] fp32 final states; NULL = not written.  May
 *               alias S0 (then S0 is overwritten with the final state).
 *   workspace   device buffer of at least the queried size (may be NULL
 *               when that size is 0).
 *
 * T = 0 (or an empty sequence) writes no o and copies S0 (or zeros) to S_T.
 * Compiled instances (d_k, d_v, chunk, io_dtype):
 *   (64, 64, 64, BF16), (128, 128, 64, BF16) -- MFMA kernels;
 *   (16|32|64, same, 16|32|64, F32)          -- fp32 kernels.
 * Returns a gdn_status. */
int gdn_chunk_fwd(const gdn_shape *shape,
                  const void *q, const void *k, const void *v,
                  const float *log_alpha, const float *beta,
                  const float *S0, const int32_t *cu_seqlens,
                  void *o, float *S_T,
                  void *workspace, size_t workspace_bytes,
                  void *stream);

/* Bytes of device workspace gdn_chunk_bwd needs for `shape` (written to
 * *bytes): per chunk of 64 tokens and head, fp32 copies of T and P, the
 * state entering the chunk and its gradient, and five 64 x d intermediates
 * -- about (2 d^2 + 5 * 64 d + 2 * 64^2) * 4 bytes (288 KiB at d = 128).
 * Returns a gdn_status (the backward's own supported set, see below). */
int gdn_chunk_bwd_workspace_size(const gdn_shape *shape, size_t *bytes);

/* Backward pass of gdn_chunk_fwd: the gradients of
 *     L = sum_t <dO_t, o_t> + sum_units <dS_T, S_T>
 * with respect to q, k, v, log_alpha, beta and S0, for the same shape and
 * inputs.  The pages name a gate-aware backward pass for the chunkwise
 * algorithm ("Gated DeltaNet-2: Decoupling Erase and Write in Linear
 * Attention", abstract) but print none; the gradient is the one of the
 * forward defined above, computed chunkwise (state gradients in reverse
 * chunk order, each chunk's gradients from the state entering it and the
 * gradient of the state leaving it) in fp32.
 *
 *   q, k, v, log_alpha, beta, S0, cu_seqlens   as in gdn_chunk_fwd
 *   dO          [B, T, H, d_v]  o_dtype, gradient of o
 *   dS_T        [U, H, d_v, d_k] fp32 gradient of the final states; NULL = 0
 *   dq, dk      [B, T, H, d_k]  o_dtype outputs
 *   dv          [B, T, H, d_v]  o_dtype output
 *   dlog_alpha, dbeta [B, T, H] fp32 outputs
 *   dS0         [U, H, d_v, d_k] fp32 output; NULL = not written
 *   workspace   device buffer of at least gdn_chunk_bwd_workspace_size bytes
 * No output may alias an input.  Supported: chunk 64, prologue 0, d_k = d_v
 * in {64, 128} with bf16 inputs or d_k = d_v = 64 with fp32 inputs.
 * Returns a gdn_status. */
int gdn_chunk_bwd(const gdn_shape *shape,
                  const void *q, const void *k, const void *v,
                  const float *log_alpha, const float *beta,
                  const float *S0, const int32_t *cu_seqlens,
                  const void *dO, const float *dS_T,
                  void *dq, void *dk, void *dv,
                  float *dlog_alpha, float *dbeta, float *dS0,
                  void *workspace, size_t workspace_bytes,
                  void *stream);

/* Bytes of device workspace gdn_kda_fwd needs for `shape`: per chunk of 64
 * tokens and head, fp32 T and P (64 x 64), K o e^G, Q o e^G and
 * K o e^{G_n - G} (64 x d), e^{G_n} (d) and beta (64) -- about
 * (2 * 64^2 + 3 * 64 d + d + 64) * 4 bytes (128 KiB at d = 128).
 * Returns a gdn_status. */
int gdn_kda_fwd_workspace_size(const gdn_shape *shape, size_t *bytes);

/* Chunkwise forward of the delta rule with channel-wise decay (KDA).  The
 * pages describe it only in words ("Gated DeltaNet-2: Decoupling Erase and
 * Write in Linear Attention", abstract: the delta rule with channel-wise
 * decay, reducing to Gated DeltaNet when the decay is a scalar); the rule
 * computed here lets the decay act on the key channels before the update:
 *
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,     alpha_t in (0,1]^{d_k}
 *
 * with every argument as in gdn_chunk_fwd except
 *   log_alpha   [B, T, H, d_k]  fp32, log of the channel-wise gate
 * and a required workspace (gdn_kda_fwd_workspace_size).  With equal
 * channels it computes gdn_chunk_fwd's rule.  fp32 arithmetic throughout.
 * Supported: chunk 64, prologue 0, d_k = d_v in {64, 128} with bf16 inputs
 * or d_k = d_v = 64 with fp32 inputs.  Returns a gdn_status. */
int gdn_kda_fwd(const gdn_shape *shape,
                const void *q, const void *k, const void *v,
                const float *log_alpha, const float *beta,
                const float *S0, const int32_t *cu_seqlens,
                void *o, float *S_T,
                void *workspace, size_t workspace_bytes,
                void *stream);

/* gdn_kda_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace taken from a device
 * array inside the library (64 MiB, one per GPU the library runs on, held
 * until the process ends) instead of a caller buffer.  Every argument as in
 * gdn_kda_fwd; the caller still supplies o and S_T.  Shapes whose
 * gdn_kda_fwd_workspace_size exceeds gdn_kda_fwd_noalloc_max_workspace()
 * are rejected with GDN_ERR_WORKSPACE before anything is enqueued (64 MiB
 * holds 512 chunk-heads at d = 128, e.g. one sequence of 2048 tokens with 16
 * heads).  The device current on the calling thread must be the one the
 * pointers and the stream belong to; the first call on a device looks up
 * that device's copy of the array (no allocation).  Calls on one GPU share
 * its array: calls that overlap in time on one GPU (different streams, or
 * host threads) race and give wrong results; calls ordered on one stream
 * are safe.  Allocates nothing.  Returns a gdn_status. */
int gdn_kda_fwd_noalloc(const gdn_shape *shape,
                        const void *q, const void *k, const void *v,
                        const float *log_alpha, const float *beta,
                        const float *S0, const int32_t *cu_seqlens,
                        void *o, float *S_T,
                        void *stream);

/* Size in bytes of the device array gdn_kda_fwd_noalloc uses as workspace. */
size_t gdn_kda_fwd_noalloc_max_workspace(void);

/* Bytes of device workspace gdn_gdn2_fwd needs for `shape`: per chunk of 64
 * tokens and head, two 64 x 64 and four 64 x d fp32 blocks and e^{G_n}
 * (about 160 KiB at d = 128).  Returns a gdn_status. */
int gdn_gdn2_fwd_workspace_size(const gdn_shape *shape, size_t *bytes);

/* Chunkwise forward of Gated DeltaNet-2: channel-wise decay, a channel-wise
 * erase gate on the key side and a channel-wise write gate on the value
 * side.  The pages describe it in words only ("Gated DeltaNet-2: Decoupling
 * Erase and Write in Linear Attention", abstract: the delta rule's scalar
 * gate split into an erase and a write gate, reducing to KDA when both are
 * one scalar); the rule computed here:
 *
 *     S~  = S_{t-1} Diag(alpha_t)
 *     S_t = S~ - (S~ k_t)(b_t o k_t)^T + (w_t o v_t) k_t^T,   o_t = S_t q_t
 *
 * with every argument as in gdn_kda_fwd except
 *   erase   [B, T, H, d_k]  fp32, b_t
 *   write   [B, T, H, d_v]  fp32, w_t
 * and its own workspace (gdn_gdn2_fwd_workspace_size).  With b_t and w_t
 * equal to beta_t in every channel it computes gdn_kda_fwd's rule.  fp32
 * arithmetic throughout.  Supported: chunk 64, prologue 0, d_k = d_v in
 * {64, 128} with bf16 inputs or d_k = d_v = 64 with fp32 inputs.  Returns a
 * gdn_status. */
int gdn_gdn2_fwd(const gdn_shape *shape,
                 const void *q, const void *k, const void *v,
                 const float *log_alpha, const float *erase, const float *write,
                 const float *S0, const int32_t *cu_seqlens,
                 void *o, float *S_T,
                 void *workspace, size_t workspace_bytes,
                 void *stream);

/* One recurrent decode step of the same rule for every (b, h): reads one
 * token, updates the state in place and returns the read-out -- the
 * constant-memory decoding of "Gated DeltaNet-2: Decoupling Erase and Write
 * in Linear Attention" (abstract), for the scalar-gate rule above.
 *
 *   q, k       [B, H, d_k]        io_dtype
 *   v          [B, H, d_v]        io_dtype
 *   log_alpha  [B, H]             fp32
 *   beta       [B, H]             fp32
 *   S          [B, H, d_v, d_k]   fp32, read and overwritten in place
 *   o          [B, H, d_v]        o_dtype output; must not alias S
 *   prologue   OR of gdn_prologue flags, as in gdn_shape
 *
 * Supported: d_k = 128 or 64, any d_v >= 1; either dtype for the inputs and
 * for o.  Returns a gdn_status. */
int gdn_step(int B, int H, int d_k, int d_v, int io_dtype, int o_dtype, int prologue,
             const void *q, const void *k, const void *v,
             const float *log_alpha, const float *beta,
             float *S, void *o, void *stream);

/* Message describing the last error on the calling thread ("" if none). */
const char *gdn_last_error(void);

/* Library version string, e.g. "gdn-mi355x 0.1.0 (gfx950)". */
const char *gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
