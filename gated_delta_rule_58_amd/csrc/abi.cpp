// C ABI of libgdn.so: host-side validation and kernel dispatch.  Every check
// runs before anything is enqueued, so a rejected call has no effect.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

namespace gdn {
hipError_t launch_step(int B, int H, int DK, int DV, bool io_bf16, bool o_bf16,
                       bool norm_qk, bool gates, const void *q, const void *k, const void *v,
                       const float *la, const float *beta, float *S, void *o, hipStream_t st);
bool chunk_f32_supported(int dk, int dv, int chunk);
hipError_t launch_chunk_f32(int units, int T, int H, int dk, int chunk, bool o_bf16,
                            bool norm_qk, bool gates,
                            const int32_t *cu, const void *q, const void *k, const void *v,
                            const float *la, const float *beta, const float *S0, void *o,
                            float *S_T, hipStream_t st);
bool chunk_mfma_supported(int dk, int dv, int chunk);
hipError_t launch_chunk_mfma(int units, int T, int H, int dk, bool o_bf16, bool norm_qk,
                             bool gates, const int32_t *cu, const void *q, const void *k,
                             const void *v, const float *la, const float *beta,
                             const float *S0, void *o, float *S_T, hipStream_t st);
bool chunk_bwd_supported(int dk, int dv, int chunk, bool io_bf16);
size_t chunk_bwd_ws_bytes(int units, int T, int H, int d, bool varlen);
hipError_t launch_chunk_bwd(int units, int T, int H, int d, bool io_bf16, bool g_bf16,
                            const int32_t *cu, const void *q, const void *k, const void *v,
                            const float *la, const float *beta, const float *S0,
                            const void *dO, const float *dST, void *dq, void *dk, void *dv,
                            float *dla, float *dbeta, float *dS0, void *ws, hipStream_t st);
bool kda_supported(int dk, int dv, int chunk, bool io_bf16);
size_t kda_ws_bytes(int units, int T, int H, int d, bool varlen);
size_t kda_scratch_bytes();
hipError_t kda_scratch_ptr(void **ptr);
hipError_t launch_kda_fwd(int units, int T, int H, int d, bool io_bf16, bool o_bf16,
                          const int32_t *cu, const void *q, const void *k, const void *v,
                          const float *la, const float *beta, const float *S0, void *o,
                          float *S_T, void *ws, hipStream_t st);
bool gdn2_supported(int dk, int dv, int chunk, bool io_bf16);
size_t gdn2_ws_bytes(int units, int T, int H, int d, bool varlen);
hipError_t launch_gdn2_fwd(int units, int T, int H, int d, bool io_bf16, bool o_bf16,
                           const int32_t *cu, const void *q, const void *k, const void *v,
                           const float *la, const float *erase, const float *write,
                           const float *S0, void *o, float *S_T, void *ws, hipStream_t st);
}  // namespace gdn

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return GDN_OK;
}

bool misaligned(const void *p) {
    return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0;
}

bool valid_dtype(int d) { return d == GDN_F32 || d == GDN_BF16; }

bool valid_prologue(int p) { return (p & ~(GDN_PROLOGUE_NORM_QK | GDN_PROLOGUE_GATES)) == 0; }

// Shape checks shared by the workspace query and the forward call.
int check_shape(const gdn_shape *s) {
    if (!s) return fail(GDN_ERR_INVALID_ARG, "shape is NULL");
    if (s->B <= 0 || s->H <= 0 || s->T < 0 || s->d_k <= 0 || s->d_v <= 0 || s->chunk <= 0)
        return fail(GDN_ERR_INVALID_ARG,
                    "bad dimensions B=%d T=%d H=%d d_k=%d d_v=%d chunk=%d (need B,H,d_k,d_v,chunk > 0, T >= 0)",
                    s->B, s->T, s->H, s->d_k, s->d_v, s->chunk);
    if (s->n_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "n_seqs=%d is negative", s->n_seqs);
    if (s->n_seqs > 0 && s->B != 1)
        return fail(GDN_ERR_INVALID_ARG, "packed sequences (n_seqs=%d) need B == 1, got B=%d",
                    s->n_seqs, s->B);
    if (!valid_dtype(s->io_dtype) || !valid_dtype(s->o_dtype))
        return fail(GDN_ERR_INVALID_ARG, "io_dtype=%d / o_dtype=%d is not a gdn_dtype",
                    s->io_dtype, s->o_dtype);
    if (!valid_prologue(s->prologue))
        return fail(GDN_ERR_INVALID_ARG, "prologue=%d has bits outside gdn_prologue",
                    s->prologue);
    const long units = s->n_seqs > 0 ? s->n_seqs : s->B;
    if ((long)units * s->H > (1L << 28))
        return fail(GDN_ERR_INVALID_ARG, "units x heads = %ld is too large", units * (long)s->H);
    if (s->H > 32768)
        return fail(GDN_ERR_UNSUPPORTED, "H=%d exceeds the supported 32768 heads", s->H);
    const bool ok_inst = s->io_dtype == GDN_BF16
                             ? gdn::chunk_mfma_supported(s->d_k, s->d_v, s->chunk)
                             : gdn::chunk_f32_supported(s->d_k, s->d_v, s->chunk);
    if (!ok_inst)
        return fail(GDN_ERR_UNSUPPORTED,
                    "no kernel for d_k=%d d_v=%d chunk=%d io_dtype=%s (bf16: d_k=d_v in {64,128}, "
                    "chunk 64; f32: d_k=d_v in {16,32,64}, chunk in {16,32,64})",
                    s->d_k, s->d_v, s->chunk, s->io_dtype == GDN_BF16 ? "bf16" : "f32");
    return GDN_OK;
}

// Shape checks shared by the backward and the channel-wise decay forward
// (their own supported sets, no prologue).
int check_fp32tile_shape(const gdn_shape *s, int kind) {   // 0 bwd, 1 KDA, 2 GDN-2
    const char *entry = kind == 2 ? "gdn_gdn2_fwd" : kind == 1 ? "gdn_kda_fwd" : "gdn_chunk_bwd";
    if (!s) return fail(GDN_ERR_INVALID_ARG, "shape is NULL");
    if (s->B <= 0 || s->H <= 0 || s->T < 0 || s->d_k <= 0 || s->d_v <= 0 || s->chunk <= 0)
        return fail(GDN_ERR_INVALID_ARG,
                    "bad dimensions B=%d T=%d H=%d d_k=%d d_v=%d chunk=%d (need B,H,d_k,d_v,chunk > 0, T >= 0)",
                    s->B, s->T, s->H, s->d_k, s->d_v, s->chunk);
    if (s->n_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "n_seqs=%d is negative", s->n_seqs);
    if (s->n_seqs > 0 && s->B != 1)
        return fail(GDN_ERR_INVALID_ARG, "packed sequences (n_seqs=%d) need B == 1, got B=%d",
                    s->n_seqs, s->B);
    if (!valid_dtype(s->io_dtype) || !valid_dtype(s->o_dtype))
        return fail(GDN_ERR_INVALID_ARG, "io_dtype=%d / o_dtype=%d is not a gdn_dtype",
                    s->io_dtype, s->o_dtype);
    if (!valid_prologue(s->prologue))
        return fail(GDN_ERR_INVALID_ARG, "prologue=%d has bits outside gdn_prologue",
                    s->prologue);
    if (s->prologue != 0)
        return fail(GDN_ERR_UNSUPPORTED, "%s takes no input prologue (prologue=%d)",
                    entry, s->prologue);
    if (s->H > 32768)   // keeps the 32-bit row offsets of the kernels' buffer stores in range
        return fail(GDN_ERR_UNSUPPORTED, "H=%d exceeds the supported 32768 heads", s->H);
    const long units = s->n_seqs > 0 ? s->n_seqs : s->B;
    if ((long)units * s->H > (1L << 24) || (long)s->T * s->H > (1L << 31) / 64)
        return fail(GDN_ERR_INVALID_ARG,
                    "problem too large for %s (units x heads = %ld, T x heads = %ld)", entry,
                    units * (long)s->H, (long)s->T * s->H);
    const bool bf = s->io_dtype == GDN_BF16;
    const bool okk = kind == 2 ? gdn::gdn2_supported(s->d_k, s->d_v, s->chunk, bf)
                     : kind == 1 ? gdn::kda_supported(s->d_k, s->d_v, s->chunk, bf)
                               : gdn::chunk_bwd_supported(s->d_k, s->d_v, s->chunk, bf);
    if (!okk)
        return fail(GDN_ERR_UNSUPPORTED,
                    "no %s kernel for d_k=%d d_v=%d chunk=%d io_dtype=%s (bf16: d_k=d_v in "
                    "{64,128}; f32: d_k=d_v=64; chunk 64)",
                    entry, s->d_k, s->d_v, s->chunk,
                    s->io_dtype == GDN_BF16 ? "bf16" : "f32");
    return GDN_OK;
}
int check_bwd_shape(const gdn_shape *s) { return check_fp32tile_shape(s, 0); }

}  // namespace

extern "C" {

const char *gdn_last_error(void) { return g_last_error.c_str(); }

const char *gdn_version(void) { return "gdn-mi355x 0.1.0 (gfx950)"; }

int gdn_chunk_fwd_workspace_size(const gdn_shape *shape, size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_ARG, "bytes is NULL");
    const int rc = check_shape(shape);
    if (rc != GDN_OK) return rc;
    *bytes = 0;
    return ok();
}

int gdn_chunk_fwd(const gdn_shape *s, const void *q, const void *k, const void *v,
                  const float *log_alpha, const float *beta, const float *S0,
                  const int32_t *cu_seqlens, void *o, float *S_T, void *workspace,
                  size_t workspace_bytes, void *stream) {
    int rc = check_shape(s);
    if (rc != GDN_OK) return rc;
    if (s->n_seqs > 0 && !cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "n_seqs=%d but cu_seqlens is NULL", s->n_seqs);
    if (s->n_seqs == 0 && cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens given but n_seqs is 0");
    if (s->T > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, log_alpha, beta and o are required when T > 0");
    const void *ptrs[] = {q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, workspace};
    const char *names[] = {"q", "k", "v", "log_alpha", "beta", "S0", "cu_seqlens", "o", "S_T",
                           "workspace"};
    for (int i = 0; i < 10; ++i)
        if (misaligned(ptrs[i]))
            return fail(GDN_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    if (o && (o == q || o == k || o == v))
        return fail(GDN_ERR_INVALID_ARG, "o must not alias q, k or v");
    size_t need = 0;
    gdn_chunk_fwd_workspace_size(s, &need);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (s->T == 0 && !S_T) return ok();   // nothing to produce

    const int units = s->n_seqs > 0 ? s->n_seqs : s->B;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool o_bf16 = s->o_dtype == GDN_BF16;
    const bool norm_qk = (s->prologue & GDN_PROLOGUE_NORM_QK) != 0;
    const bool gates = (s->prologue & GDN_PROLOGUE_GATES) != 0;
    hipError_t e;
    if (s->io_dtype == GDN_BF16)
        e = gdn::launch_chunk_mfma(units, s->T, s->H, s->d_k, o_bf16, norm_qk, gates, cu_seqlens,
                                   q, k, v, log_alpha, beta, S0, o, S_T, st);
    else
        e = gdn::launch_chunk_f32(units, s->T, s->H, s->d_k, s->chunk, o_bf16, norm_qk, gates,
                                  cu_seqlens, q, k, v, log_alpha, beta, S0, o, S_T, st);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gdn_chunk_bwd_workspace_size(const gdn_shape *shape, size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_ARG, "bytes is NULL");
    const int rc = check_bwd_shape(shape);
    if (rc != GDN_OK) return rc;
    const int units = shape->n_seqs > 0 ? shape->n_seqs : shape->B;
    *bytes = gdn::chunk_bwd_ws_bytes(units, shape->T, shape->H, shape->d_k, shape->n_seqs > 0);
    return ok();
}

int gdn_chunk_bwd(const gdn_shape *s, const void *q, const void *k, const void *v,
                  const float *log_alpha, const float *beta, const float *S0,
                  const int32_t *cu_seqlens, const void *dO, const float *dS_T, void *dq,
                  void *dk, void *dv, float *dlog_alpha, float *dbeta, float *dS0,
                  void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_bwd_shape(s);
    if (rc != GDN_OK) return rc;
    if (s->n_seqs > 0 && !cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "n_seqs=%d but cu_seqlens is NULL", s->n_seqs);
    if (s->n_seqs == 0 && cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens given but n_seqs is 0");
    if (s->T > 0 && (!q || !k || !v || !log_alpha || !beta || !dO || !dq || !dk || !dv ||
                     !dlog_alpha || !dbeta))
        return fail(GDN_ERR_INVALID_ARG,
                    "q, k, v, log_alpha, beta, dO and every token gradient are required when T > 0");
    const void *ptrs[] = {q, k, v, log_alpha, beta, S0, cu_seqlens, dO, dS_T, dq, dk, dv,
                          dlog_alpha, dbeta, dS0, workspace};
    const char *names[] = {"q", "k", "v", "log_alpha", "beta", "S0", "cu_seqlens", "dO", "dS_T",
                           "dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0", "workspace"};
    for (int i = 0; i < 16; ++i)
        if (misaligned(ptrs[i]))
            return fail(GDN_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    const void *ins[] = {q, k, v, log_alpha, beta, S0, dO, dS_T};
    const void *outs[] = {dq, dk, dv, dlog_alpha, dbeta, dS0};
    for (const void *o : outs)
        for (const void *in : ins)
            if (o && o == in) return fail(GDN_ERR_INVALID_ARG, "a gradient output aliases an input");
    size_t need = 0;
    gdn_chunk_bwd_workspace_size(s, &need);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (need > 0 && !workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL");
    const int units = s->n_seqs > 0 ? s->n_seqs : s->B;
    const hipError_t e = gdn::launch_chunk_bwd(
        units, s->T, s->H, s->d_k, s->io_dtype == GDN_BF16, s->o_dtype == GDN_BF16, cu_seqlens, q,
        k, v, log_alpha, beta, S0, dO, dS_T, dq, dk, dv, dlog_alpha, dbeta, dS0, workspace,
        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gdn_kda_fwd_workspace_size(const gdn_shape *shape, size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_ARG, "bytes is NULL");
    const int rc = check_fp32tile_shape(shape, 1);
    if (rc != GDN_OK) return rc;
    const int units = shape->n_seqs > 0 ? shape->n_seqs : shape->B;
    *bytes = gdn::kda_ws_bytes(units, shape->T, shape->H, shape->d_k, shape->n_seqs > 0);
    return ok();
}

}  // extern "C"

namespace {
// Argument checks of gdn_kda_fwd and gdn_kda_fwd_noalloc (all but the workspace).
int check_kda_args(const gdn_shape *s, const void *q, const void *k, const void *v,
                   const float *log_alpha, const float *beta, const float *S0,
                   const int32_t *cu_seqlens, void *o, float *S_T, void *workspace) {
    int rc = check_fp32tile_shape(s, 1);
    if (rc != GDN_OK) return rc;
    if (s->n_seqs > 0 && !cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "n_seqs=%d but cu_seqlens is NULL", s->n_seqs);
    if (s->n_seqs == 0 && cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens given but n_seqs is 0");
    if (s->T > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, log_alpha, beta and o are required when T > 0");
    const void *ptrs[] = {q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, workspace};
    const char *names[] = {"q", "k", "v", "log_alpha", "beta", "S0", "cu_seqlens", "o", "S_T",
                           "workspace"};
    for (int i = 0; i < 10; ++i)
        if (misaligned(ptrs[i]))
            return fail(GDN_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    if (o && (o == q || o == k || o == v))
        return fail(GDN_ERR_INVALID_ARG, "o must not alias q, k or v");
    return GDN_OK;
}
}  // namespace

extern "C" {

int gdn_kda_fwd(const gdn_shape *s, const void *q, const void *k, const void *v,
                const float *log_alpha, const float *beta, const float *S0,
                const int32_t *cu_seqlens, void *o, float *S_T, void *workspace,
                size_t workspace_bytes, void *stream) {
    int rc = check_kda_args(s, q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, workspace);
    if (rc != GDN_OK) return rc;
    size_t need = 0;
    gdn_kda_fwd_workspace_size(s, &need);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (need > 0 && !workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL");
    const int units = s->n_seqs > 0 ? s->n_seqs : s->B;
    const hipError_t e = gdn::launch_kda_fwd(
        units, s->T, s->H, s->d_k, s->io_dtype == GDN_BF16, s->o_dtype == GDN_BF16, cu_seqlens, q,
        k, v, log_alpha, beta, S0, o, S_T, workspace, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t gdn_kda_fwd_noalloc_max_workspace(void) { return gdn::kda_scratch_bytes(); }

int gdn_kda_fwd_noalloc(const gdn_shape *s, const void *q, const void *k, const void *v,
                        const float *log_alpha, const float *beta, const float *S0,
                        const int32_t *cu_seqlens, void *o, float *S_T, void *stream) {
    int rc = check_kda_args(s, q, k, v, log_alpha, beta, S0, cu_seqlens, o, S_T, nullptr);
    if (rc != GDN_OK) return rc;
    size_t need = 0;
    gdn_kda_fwd_workspace_size(s, &need);
    const size_t cap = gdn::kda_scratch_bytes();
    if (need > cap)
        return fail(GDN_ERR_WORKSPACE,
                    "gdn_kda_fwd_noalloc: this shape needs %zu bytes of workspace, the library's "
                    "device scratch holds %zu; use gdn_kda_fwd with a caller workspace",
                    need, cap);
    void *ws = nullptr;
    hipError_t e = gdn::kda_scratch_ptr(&ws);
    if (e != hipSuccess)
        return fail(GDN_ERR_HIP, "device scratch address unavailable: %s", hipGetErrorString(e));
    const int units = s->n_seqs > 0 ? s->n_seqs : s->B;
    e = gdn::launch_kda_fwd(units, s->T, s->H, s->d_k, s->io_dtype == GDN_BF16,
                            s->o_dtype == GDN_BF16, cu_seqlens, q, k, v, log_alpha, beta, S0, o,
                            S_T, ws, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gdn_gdn2_fwd_workspace_size(const gdn_shape *shape, size_t *bytes) {
    if (!bytes) return fail(GDN_ERR_INVALID_ARG, "bytes is NULL");
    const int rc = check_fp32tile_shape(shape, 2);
    if (rc != GDN_OK) return rc;
    const int units = shape->n_seqs > 0 ? shape->n_seqs : shape->B;
    *bytes = gdn::gdn2_ws_bytes(units, shape->T, shape->H, shape->d_k, shape->n_seqs > 0);
    return ok();
}

int gdn_gdn2_fwd(const gdn_shape *s, const void *q, const void *k, const void *v,
                 const float *log_alpha, const float *erase, const float *write,
                 const float *S0, const int32_t *cu_seqlens, void *o, float *S_T,
                 void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_fp32tile_shape(s, 2);
    if (rc != GDN_OK) return rc;
    if (s->n_seqs > 0 && !cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "n_seqs=%d but cu_seqlens is NULL", s->n_seqs);
    if (s->n_seqs == 0 && cu_seqlens)
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens given but n_seqs is 0");
    if (s->T > 0 && (!q || !k || !v || !log_alpha || !erase || !write || !o))
        return fail(GDN_ERR_INVALID_ARG,
                    "q, k, v, log_alpha, erase, write and o are required when T > 0");
    const void *ptrs[] = {q, k, v, log_alpha, erase, write, S0, cu_seqlens, o, S_T, workspace};
    const char *names[] = {"q", "k", "v", "log_alpha", "erase", "write", "S0", "cu_seqlens",
                           "o", "S_T", "workspace"};
    for (int i = 0; i < 11; ++i)
        if (misaligned(ptrs[i]))
            return fail(GDN_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    if (o && (o == q || o == k || o == v))
        return fail(GDN_ERR_INVALID_ARG, "o must not alias q, k or v");
    size_t need = 0;
    gdn_gdn2_fwd_workspace_size(s, &need);
    if (workspace_bytes < need)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (need > 0 && !workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL");
    const int units = s->n_seqs > 0 ? s->n_seqs : s->B;
    const hipError_t e = gdn::launch_gdn2_fwd(
        units, s->T, s->H, s->d_k, s->io_dtype == GDN_BF16, s->o_dtype == GDN_BF16, cu_seqlens, q,
        k, v, log_alpha, erase, write, S0, o, S_T, workspace,
        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gdn_step(int B, int H, int d_k, int d_v, int io_dtype, int o_dtype, int prologue,
             const void *q, const void *k, const void *v, const float *log_alpha,
             const float *beta, float *S, void *o, void *stream) {
    if (B <= 0 || H <= 0 || d_k <= 0 || d_v <= 0)
        return fail(GDN_ERR_INVALID_ARG, "bad dimensions B=%d H=%d d_k=%d d_v=%d", B, H, d_k, d_v);
    if (!valid_dtype(io_dtype) || !valid_dtype(o_dtype))
        return fail(GDN_ERR_INVALID_ARG, "io_dtype=%d / o_dtype=%d is not a gdn_dtype", io_dtype,
                    o_dtype);
    if (!valid_prologue(prologue))
        return fail(GDN_ERR_INVALID_ARG, "prologue=%d has bits outside gdn_prologue", prologue);
    if ((long)B * H > (1L << 30))
        return fail(GDN_ERR_INVALID_ARG, "B x H = %ld is too large", (long)B * H);
    if (d_k != 64 && d_k != 128)
        return fail(GDN_ERR_UNSUPPORTED, "no decode kernel for d_k=%d (64 or 128)", d_k);
    if (!q || !k || !v || !log_alpha || !beta || !S || !o)
        return fail(GDN_ERR_INVALID_ARG, "every pointer of gdn_step is required");
    const void *ptrs[] = {q, k, v, log_alpha, beta, S, o};
    const char *names[] = {"q", "k", "v", "log_alpha", "beta", "S", "o"};
    for (int i = 0; i < 7; ++i)
        if (misaligned(ptrs[i]))
            return fail(GDN_ERR_ALIGNMENT, "%s=%p is not 16-byte aligned", names[i], ptrs[i]);
    if (o == (void *)S) return fail(GDN_ERR_INVALID_ARG, "o must not alias S");
    const hipError_t e =
        gdn::launch_step(B, H, d_k, d_v, io_dtype == GDN_BF16, o_dtype == GDN_BF16,
                         (prologue & GDN_PROLOGUE_NORM_QK) != 0,
                         (prologue & GDN_PROLOGUE_GATES) != 0, q, k, v, log_alpha, beta, S, o,
                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
