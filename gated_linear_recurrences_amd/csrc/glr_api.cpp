// C ABI of the library: argument validation, status mapping and dispatch to
// the kernels. No allocation (scratch memory is the caller's workspace), no
// global mutable state besides the thread-local text of the last error.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <limits>
#include <cstdio>
#include <cstring>

#include "glr.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[256] = "";

la_status fail(la_status st, const char* fmt, const char* what) {
    std::snprintf(g_last_error, sizeof(g_last_error), fmt, what);
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<std::uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// A pointer that is dereferenced must be non-null and 16-byte aligned.
la_status check_ptr(const void* p, bool used, bool optional, const char* name) {
    if (p == nullptr) {
        if (used && !optional) return fail(LA_ERR_INVALID, "%s is NULL", name);
        return LA_OK;
    }
    if (!aligned16(p)) return fail(LA_ERR_INVALID, "%s is not 16-byte aligned", name);
    return LA_OK;
}

// Sizes, dtype and (unless `pointers` is false: the workspace query) the pointers of a chunk call.
la_status check_chunk_args(glr::Variant variant, const glr::ChunkArgs& a, int dtype, bool pointers = true) {
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "%s", "unknown dtype");
    if (a.B < 0 || a.H < 0 || a.T < 0) return fail(LA_ERR_INVALID, "%s", "negative B, H or T");
    if (a.chunk < 1) return fail(LA_ERR_INVALID, "%s", "chunk < 1");
    if (a.dk < 1 || a.dv < 1) return fail(LA_ERR_INVALID, "%s", "d_k and d_v must be >= 1");
    if (!supported_dim(a.dk) || !supported_dim(a.dv))
        return fail(LA_ERR_UNSUPPORTED, "%s", "d_k and d_v must be 16, 32, 64 or 128");
    if (a.chunk != 16 && a.chunk != 32 && a.chunk != 64)
        return fail(LA_ERR_UNSUPPORTED, "%s", "chunk must be 16, 32 or 64");
    const bool heads = pointers && a.B > 0 && a.H > 0;
    const bool tokens = heads && a.T > 0;
    la_status st;
    if ((st = check_ptr(a.q, tokens, false, "q")) != LA_OK) return st;
    if ((st = check_ptr(a.k, tokens, false, "k")) != LA_OK) return st;
    if ((st = check_ptr(a.v, tokens, false, "v")) != LA_OK) return st;
    if ((st = check_ptr(a.o, tokens, false, "o")) != LA_OK) return st;
    // retention's per-head decay is read by every launched workgroup, also when T == 0
    if ((st = check_ptr(a.gate, variant == glr::kRetention ? heads : tokens, false,
                        variant == glr::kRetention ? "log_gamma" : "log_alpha")) != LA_OK)
        return st;
    if (variant == glr::kGDelta && (st = check_ptr(a.beta, tokens, false, "beta")) != LA_OK) return st;
    if ((st = check_ptr(a.s0, heads, true, "s0")) != LA_OK) return st;
    if ((st = check_ptr(a.s_out, heads, true, "s_out")) != LA_OK) return st;
    const int64_t elems = static_cast<int64_t>(a.B) * a.H * a.T * (a.dk > a.dv ? a.dk : a.dv);
    if (elems > (static_cast<int64_t>(1) << 40)) return fail(LA_ERR_INVALID, "%s", "tensor too large");
    if (static_cast<int64_t>(a.B) * a.H > (static_cast<int64_t>(1) << 24))
        return fail(LA_ERR_UNSUPPORTED, "%s", "B * H must be below 2^24");
    const int64_t chunks = static_cast<int64_t>(a.B) * a.H * ((static_cast<int64_t>(a.T) + a.chunk - 1) / a.chunk);
    if (chunks >= (static_cast<int64_t>(1) << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s", "B * H * ceil(T / chunk) must be below 2^31");
    return LA_OK;
}

la_status run_chunk(glr::Variant variant, const glr::ChunkArgs& a, la_dtype dtype, size_t ws_bytes,
                    void* stream) {
    la_status st = check_chunk_args(variant, a, dtype);
    if (st != LA_OK) return st;
    const size_t need = glr::chunk_workspace_bytes(variant, a, dtype == LA_BF16);
    if (need > 0) {
        if (a.ws == nullptr) return fail(LA_ERR_INVALID, "%s", "workspace is NULL");
        if (!aligned16(a.ws)) return fail(LA_ERR_INVALID, "%s", "workspace is not 16-byte aligned");
        if (ws_bytes < need) return fail(LA_ERR_INVALID, "%s", "workspace too small");
    }
    if (a.B == 0 || a.H == 0) return LA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = (dtype == LA_BF16) ? glr::launch_chunk_bf16(variant, a, s)
                                              : glr::launch_chunk_f32(variant, a, s);
    if (err != hipSuccess) return fail(LA_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
    return LA_OK;
}

}  // namespace

namespace glr {
int report_error(int status, const char* message) {
    return fail(static_cast<la_status>(status), "%s", message);
}
int check_chunk_call(Variant variant, const ChunkArgs& a, int dtype) { return check_chunk_args(variant, a, dtype); }
}  // namespace glr

extern "C" {

la_status la_chunk_workspace_size(la_variant variant, int B, int H, int T, int dk, int dv, int chunk,
                                  la_dtype dtype, size_t* bytes) {
    if (bytes == nullptr) return fail(LA_ERR_INVALID, "%s", "bytes is NULL");
    *bytes = 0;
    if (variant != LA_RETENTION && variant != LA_GLA && variant != LA_GDELTA && variant != LA_MAMBA2 &&
        variant != LA_GDELTA_FUSED)
        return fail(LA_ERR_INVALID, "%s", "unknown variant");
    const glr::Variant v = variant == LA_GDELTA_FUSED ? glr::kGDelta : static_cast<glr::Variant>(variant);
    // shape checks only: pointers are not part of the query
    glr::ChunkArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     B, H, 0, dk, dv, chunk, nullptr, variant == LA_GDELTA_FUSED ? LA_FUSE_QK_SILU_L2 : 0,
                     nullptr, 0.f};
    la_status st = check_chunk_args(v, a, dtype, false);
    if (st != LA_OK) return st;
    if (T < 0) return fail(LA_ERR_INVALID, "%s", "negative B, H or T");
    a.T = T;
    const int64_t chunks = static_cast<int64_t>(B) * H * ((static_cast<int64_t>(T) + chunk - 1) / chunk);
    if (chunks >= (static_cast<int64_t>(1) << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s", "B * H * ceil(T / chunk) must be below 2^31");
    *bytes = glr::chunk_workspace_bytes(v, a, dtype == LA_BF16);
    return LA_OK;
}

la_status la_chunk_fwd(const void* q, const void* k, const void* v, const float* log_gamma,
                       const float* s0, void* o, float* s_out,
                       int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
    glr::ChunkArgs a{q, k, v, log_gamma, nullptr, s0, o, s_out, B, H, T, dk, dv, chunk, workspace};
    return run_chunk(glr::kRetention, a, dtype, workspace_bytes, stream);
}

la_status mamba2_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* s0, void* o, float* s_out,
                           int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
    glr::ChunkArgs a{q, k, v, log_alpha, nullptr, s0, o, s_out, B, H, T, dk, dv, chunk, workspace};
    return run_chunk(glr::kScalar, a, dtype, workspace_bytes, stream);
}

la_status gla_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* s0, void* o, float* s_out,
                        int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
    glr::ChunkArgs a{q, k, v, log_alpha, nullptr, s0, o, s_out, B, H, T, dk, dv, chunk, workspace};
    return run_chunk(glr::kGLA, a, dtype, workspace_bytes, stream);
}

la_status gdelta_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* s0, void* o, float* s_out,
                           int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
    glr::ChunkArgs a{q, k, v, log_alpha, beta, s0, o, s_out, B, H, T, dk, dv, chunk, workspace};
    return run_chunk(glr::kGDelta, a, dtype, workspace_bytes, stream);
}

la_status gdelta_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* beta, const float* s0, void* o, float* s_out,
                                 const float* o_norm_weight, float o_norm_eps, int fuse,
                                 int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (fuse & ~(LA_FUSE_QK_SILU_L2 | LA_FUSE_OUT_RMSNORM)) return fail(LA_ERR_INVALID, "%s", "unknown fuse flag");
    if (fuse & LA_FUSE_OUT_RMSNORM) {
        const bool rows = B > 0 && H > 0 && T > 0;
        la_status st = check_ptr(o_norm_weight, rows, false, "o_norm_weight");
        if (st != LA_OK) return st;
        if (!(o_norm_eps >= 0.f)) return fail(LA_ERR_INVALID, "%s", "o_norm_eps must be >= 0");
    }
    glr::ChunkArgs a{q, k, v, log_alpha, beta, s0, o, s_out, B, H, T, dk, dv, chunk, workspace,
                     fuse, o_norm_weight, o_norm_eps};
    return run_chunk(glr::kGDelta, a, dtype, workspace_bytes, stream);
}

la_status gla_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                              const float* s0, void* o, float* s_out, const float* o_norm_weight,
                              const float* o_norm_bias, float o_norm_eps, int fuse, int B, int H, int T, int dk,
                              int dv, int chunk, la_dtype dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (fuse & ~LA_FUSE_OUT_LAYERNORM) return fail(LA_ERR_INVALID, "%s", "unknown or unsupported fuse flag for GLA");
    if (fuse & LA_FUSE_OUT_LAYERNORM) {
        const bool rows = B > 0 && H > 0 && T > 0;
        la_status st = check_ptr(o_norm_weight, rows, false, "o_norm_weight");
        if (st != LA_OK) return st;
        if ((st = check_ptr(o_norm_bias, rows, true, "o_norm_bias")) != LA_OK) return st;
        if (!(o_norm_eps >= 0.f)) return fail(LA_ERR_INVALID, "%s", "o_norm_eps must be >= 0");
    }
    glr::ChunkArgs a{q, k, v, log_alpha, nullptr, s0, o, s_out, B, H, T, dk, dv, chunk, workspace,
                     fuse, o_norm_weight, o_norm_eps, o_norm_bias};
    return run_chunk(glr::kGLA, a, dtype, workspace_bytes, stream);
}

// Retention and the scalar decay with an output norm: RMS (weight) or layer norm (weight,
// optional bias), exactly one of the two.
static la_status run_norm_fused(glr::Variant variant, const void* q, const void* k, const void* v, const float* gate,
                                const float* s0, void* o, float* s_out, const float* w, const float* b, float eps,
                                int fuse, int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (fuse != LA_FUSE_OUT_RMSNORM && fuse != LA_FUSE_OUT_LAYERNORM)
        return fail(LA_ERR_INVALID, "%s", "fuse must be LA_FUSE_OUT_RMSNORM or LA_FUSE_OUT_LAYERNORM");
    const bool rows = B > 0 && H > 0 && T > 0;
    la_status st = check_ptr(w, rows, false, "o_norm_weight");
    if (st != LA_OK) return st;
    if (fuse == LA_FUSE_OUT_RMSNORM && b != nullptr) return fail(LA_ERR_INVALID, "%s", "the RMS norm takes no bias");
    if ((st = check_ptr(b, rows, true, "o_norm_bias")) != LA_OK) return st;
    if (!(eps >= 0.f)) return fail(LA_ERR_INVALID, "%s", "o_norm_eps must be >= 0");
    glr::ChunkArgs a{q, k, v, gate, nullptr, s0, o, s_out, B, H, T, dk, dv, chunk, workspace, fuse, w, eps, b};
    return run_chunk(variant, a, dtype, workspace_bytes, stream);
}

la_status la_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* log_gamma, const float* s0,
                             void* o, float* s_out, const float* o_norm_weight, const float* o_norm_bias,
                             float o_norm_eps, int fuse, int B, int H, int T, int dk, int dv, int chunk,
                             la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return run_norm_fused(glr::kRetention, q, k, v, log_gamma, s0, o, s_out, o_norm_weight, o_norm_bias, o_norm_eps,
                          fuse, B, H, T, dk, dv, chunk, dtype, workspace, workspace_bytes, stream);
}

la_status mamba2_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* s0, void* o, float* s_out, const float* o_norm_weight,
                                 const float* o_norm_bias, float o_norm_eps, int fuse, int B, int H, int T, int dk,
                                 int dv, int chunk, la_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return run_norm_fused(glr::kScalar, q, k, v, log_alpha, s0, o, s_out, o_norm_weight, o_norm_bias, o_norm_eps,
                          fuse, B, H, T, dk, dv, chunk, dtype, workspace, workspace_bytes, stream);
}

static la_status run_bwd(glr::Variant variant, const glr::BwdArgs& a, la_dtype dtype, size_t ws_bytes,
                         void* stream) {
    // the forward's checks on q, k, v, the gate and the dimensions (o stands for the gradients)
    glr::ChunkArgs f{a.q, a.k, a.v, a.gate, a.beta, a.s0, a.grad_q, nullptr, a.B, a.H, a.T, a.dk, a.dv, a.chunk,
                     a.ws};
    la_status st = check_chunk_args(variant, f, dtype);
    if (st != LA_OK) return st;
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s", "the backward takes bf16 storage");
    const bool heads = a.B > 0 && a.H > 0;
    const bool tokens = heads && a.T > 0;
    if ((st = check_ptr(a.dout, tokens, false, "dout")) != LA_OK) return st;
    if ((st = check_ptr(a.grad_k, tokens, false, "dk")) != LA_OK) return st;
    if ((st = check_ptr(a.grad_v, tokens, false, "dv")) != LA_OK) return st;
    if ((st = check_ptr(a.dgate, variant == glr::kRetention ? heads : tokens, false, "dgate")) != LA_OK) return st;
    if (variant == glr::kGDelta && (st = check_ptr(a.dbeta, tokens, false, "dbeta")) != LA_OK) return st;
    if ((st = check_ptr(a.ds_out, heads, true, "ds_out")) != LA_OK) return st;
    if ((st = check_ptr(a.ds0, heads, true, "ds0")) != LA_OK) return st;
    const size_t need = glr::bwd_workspace_size(variant, a);
    if (need > 0) {
        if (a.ws == nullptr) return fail(LA_ERR_INVALID, "%s", "workspace is NULL");
        if (!aligned16(a.ws)) return fail(LA_ERR_INVALID, "%s", "workspace is not 16-byte aligned");
        if (ws_bytes < need) return fail(LA_ERR_INVALID, "%s", "workspace too small");
    }
    if (!heads) return LA_OK;
    const hipError_t err = glr::launch_chunk_bwd(variant, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(LA_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
    return LA_OK;
}

la_status la_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                            float* s, void* o, int N, int H, int dk, int dv, la_dtype dtype,
                            void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "%s", "unknown dtype");
    if (N < 0 || H < 0) return fail(LA_ERR_INVALID, "%s", "negative N or H");
    if (dk < 1 || dv < 1) return fail(LA_ERR_INVALID, "%s", "d_k and d_v must be >= 1");
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s", "d_k and d_v must be 16, 32, 64 or 128");
    const bool used = N > 0 && H > 0;
    la_status st;
    if ((st = check_ptr(q, used, false, "q")) != LA_OK) return st;
    if ((st = check_ptr(k, used, false, "k")) != LA_OK) return st;
    if ((st = check_ptr(v, used, false, "v")) != LA_OK) return st;
    if ((st = check_ptr(alpha, used, false, "alpha")) != LA_OK) return st;
    if ((st = check_ptr(s, used, false, "s")) != LA_OK) return st;
    if ((st = check_ptr(o, used, false, "o")) != LA_OK) return st;
    if (static_cast<int64_t>(N) * H >= (static_cast<int64_t>(1) << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s", "N * H must be below 2^31");
    if (!used) return LA_OK;
    glr::DecodeArgs a{q, k, v, alpha, nullptr, s, o, N, H, dk, dv};
    const hipError_t err = glr::launch_decode(dtype == LA_BF16, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(LA_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
    return LA_OK;
}

la_status gdelta_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, float* s, void* o, int N, int H, int dk, int dv,
                                la_dtype dtype, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "%s", "unknown dtype");
    if (N < 0 || H < 0) return fail(LA_ERR_INVALID, "%s", "negative N or H");
    if (dk < 1 || dv < 1) return fail(LA_ERR_INVALID, "%s", "d_k and d_v must be >= 1");
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s", "d_k and d_v must be 16, 32, 64 or 128");
    const bool used = N > 0 && H > 0;
    la_status st;
    if ((st = check_ptr(q, used, false, "q")) != LA_OK) return st;
    if ((st = check_ptr(k, used, false, "k")) != LA_OK) return st;
    if ((st = check_ptr(v, used, false, "v")) != LA_OK) return st;
    if ((st = check_ptr(alpha, used, false, "alpha")) != LA_OK) return st;
    if ((st = check_ptr(beta, used, false, "beta")) != LA_OK) return st;
    if ((st = check_ptr(s, used, false, "s")) != LA_OK) return st;
    if ((st = check_ptr(o, used, false, "o")) != LA_OK) return st;
    if (static_cast<int64_t>(N) * H >= (static_cast<int64_t>(1) << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s", "N * H must be below 2^31");
    if (!used) return LA_OK;
    glr::DecodeArgs a{q, k, v, alpha, beta, s, o, N, H, dk, dv};
    const hipError_t err = glr::launch_decode(dtype == LA_BF16, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(LA_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
    return LA_OK;
}

static la_status bwd_workspace_query(glr::Variant variant, int B, int H, int T, int dk, int dv, int chunk,
                                     la_dtype dtype, size_t* bytes) {
    if (bytes == nullptr) return fail(LA_ERR_INVALID, "%s", "bytes is NULL");
    *bytes = 0;
    glr::ChunkArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     B, H, 0, dk, dv, chunk, nullptr};
    la_status st = check_chunk_args(glr::kRetention, a, dtype, false);
    if (st != LA_OK) return st;
    if (T < 0) return fail(LA_ERR_INVALID, "%s", "negative B, H or T");
    if (dtype != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "%s", "the backward takes bf16 storage");
    const int64_t chunks = static_cast<int64_t>(B) * H * ((static_cast<int64_t>(T) + chunk - 1) / chunk);
    if (chunks >= (static_cast<int64_t>(1) << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s", "B * H * ceil(T / chunk) must be below 2^31");
    glr::BwdArgs b{};
    b.B = B; b.H = H; b.T = T; b.dk = dk; b.dv = dv; b.chunk = chunk;
    *bytes = glr::bwd_workspace_size(variant, b);
    return LA_OK;
}

la_status la_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                                      size_t* bytes) {
    return bwd_workspace_query(glr::kRetention, B, H, T, dk, dv, chunk, dtype, bytes);
}

la_status gla_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                                       size_t* bytes) {
    return bwd_workspace_query(glr::kGLA, B, H, T, dk, dv, chunk, dtype, bytes);
}

la_status gdelta_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                                          size_t* bytes) {
    return bwd_workspace_query(glr::kGDelta, B, H, T, dk, dv, chunk, dtype, bytes);
}

la_status gdelta_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                           const float* s0, const void* dout, const float* ds_out, void* dq, void* dk_, void* dv_,
                           float* dlog_alpha, float* dbeta, float* ds0, int B, int H, int T, int dk, int dv, int chunk,
                           la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
    glr::BwdArgs a{q, k, v, log_alpha, s0, dout, ds_out, dq, dk_, dv_, dlog_alpha, ds0, B, H, T, dk, dv, chunk,
                   workspace, beta, dbeta};
    return run_bwd(glr::kGDelta, a, dtype, workspace_bytes, stream);
}

la_status la_chunk_bwd(const void* q, const void* k, const void* v, const float* log_gamma, const float* s0,
                       const void* dout, const float* ds_out, void* dq, void* dk_, void* dv_, float* dlog_gamma,
                       float* ds0, int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
    glr::BwdArgs a{q, k, v, log_gamma, s0, dout, ds_out, dq, dk_, dv_, dlog_gamma, ds0, B, H, T, dk, dv, chunk,
                   workspace};
    return run_bwd(glr::kRetention, a, dtype, workspace_bytes, stream);
}

la_status mamba2_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* s0,
                           const void* dout, const float* ds_out, void* dq, void* dk_, void* dv_, float* dlog_alpha,
                           float* ds0, int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
    glr::BwdArgs a{q, k, v, log_alpha, s0, dout, ds_out, dq, dk_, dv_, dlog_alpha, ds0, B, H, T, dk, dv, chunk,
                   workspace};
    return run_bwd(glr::kScalar, a, dtype, workspace_bytes, stream);
}

la_status gla_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha, const float* s0,
                        const void* dout, const float* ds_out, void* dq, void* dk_, void* dv_, float* dlog_alpha,
                        float* ds0, int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
    glr::BwdArgs a{q, k, v, log_alpha, s0, dout, ds_out, dq, dk_, dv_, dlog_alpha, ds0, B, H, T, dk, dv, chunk,
                   workspace};
    return run_bwd(glr::kGLA, a, dtype, workspace_bytes, stream);
}

la_status vla_fwd(const void* q, const void* k, const void* v, const void* u, float lambda0, const float* a0,
                  const float* s0, const float* n0, void* o, float* s_out, float* a_out, float* n_out,
                  int readout, int B, int H, int T, int dk, int dv, la_dtype dtype, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "%s", "unknown dtype");
    if (readout != LA_VLA_RATIO && readout != LA_VLA_LINEAR) return fail(LA_ERR_INVALID, "%s", "unknown readout");
    if (B < 0 || H < 0 || T < 0) return fail(LA_ERR_INVALID, "%s", "negative B, H or T");
    if (dk < 1 || dv < 1) return fail(LA_ERR_INVALID, "%s", "d_k and d_v must be >= 1");
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s", "d_k and d_v must be 16, 32, 64 or 128");
    if (a0 == nullptr && !(lambda0 > 0.f && lambda0 < std::numeric_limits<float>::infinity()))
        return fail(LA_ERR_INVALID, "%s", "lambda0 must be positive and finite when a0 is NULL");
    const bool heads = B > 0 && H > 0;
    const bool tokens = heads && T > 0;
    la_status st;
    if ((st = check_ptr(q, tokens, false, "q")) != LA_OK) return st;
    if ((st = check_ptr(k, tokens, false, "k")) != LA_OK) return st;
    if ((st = check_ptr(v, tokens, false, "v")) != LA_OK) return st;
    if ((st = check_ptr(u, tokens, false, "u")) != LA_OK) return st;
    if ((st = check_ptr(o, tokens, false, "o")) != LA_OK) return st;
    if ((st = check_ptr(a0, heads, true, "a0")) != LA_OK) return st;
    if ((st = check_ptr(s0, heads, true, "s0")) != LA_OK) return st;
    if ((st = check_ptr(s_out, heads, true, "s_out")) != LA_OK) return st;
    if ((st = check_ptr(a_out, heads, true, "a_out")) != LA_OK) return st;
    const bool ratio = readout == LA_VLA_RATIO;
    if ((st = check_ptr(n0, ratio && heads, true, "n0")) != LA_OK) return st;
    if ((st = check_ptr(n_out, ratio && heads, true, "n_out")) != LA_OK) return st;
    if (static_cast<int64_t>(B) * H >= (static_cast<int64_t>(1) << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s", "B * H must be below 2^31");
    if (!heads) return LA_OK;
    glr::VlaArgs a{q, k, v, u, a0 ? 1.f : 1.f / lambda0, a0, s0, ratio ? n0 : nullptr, o, s_out, a_out,
                   ratio ? n_out : nullptr, ratio ? 1 : 0, B, H, T, dk, dv};
    const hipError_t err = glr::launch_vla(dtype == LA_BF16, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(LA_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
    return LA_OK;
}

la_status vla_recurrent_step(const void* q, const void* k, const void* v, const void* u, float* s, float* a, float* n,
                             void* o, int readout, int N, int H, int dk, int dv, la_dtype dtype, void* stream) {
    if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "%s", "unknown dtype");
    if (readout != LA_VLA_RATIO && readout != LA_VLA_LINEAR) return fail(LA_ERR_INVALID, "%s", "unknown readout");
    if (N < 0 || H < 0) return fail(LA_ERR_INVALID, "%s", "negative N or H");
    if (dk < 1 || dv < 1) return fail(LA_ERR_INVALID, "%s", "d_k and d_v must be >= 1");
    if (!supported_dim(dk) || !supported_dim(dv))
        return fail(LA_ERR_UNSUPPORTED, "%s", "d_k and d_v must be 16, 32, 64 or 128");
    const bool used = N > 0 && H > 0;
    la_status st;
    if ((st = check_ptr(q, used, false, "q")) != LA_OK) return st;
    if ((st = check_ptr(k, used, false, "k")) != LA_OK) return st;
    if ((st = check_ptr(v, used, false, "v")) != LA_OK) return st;
    if ((st = check_ptr(u, used, false, "u")) != LA_OK) return st;
    if ((st = check_ptr(s, used, false, "s")) != LA_OK) return st;
    if ((st = check_ptr(a, used, false, "a")) != LA_OK) return st;
    const bool ratio = readout == LA_VLA_RATIO;
    if ((st = check_ptr(n, used && ratio, false, "n")) != LA_OK) return st;
    if ((st = check_ptr(o, used, false, "o")) != LA_OK) return st;
    if (static_cast<int64_t>(N) * H >= (static_cast<int64_t>(1) << 31))
        return fail(LA_ERR_UNSUPPORTED, "%s", "N * H must be below 2^31");
    if (!used) return LA_OK;
    glr::VlaArgs args{q, k, v, u, 1.f, a, s, ratio ? n : nullptr, o, s, a, ratio ? n : nullptr, ratio ? 1 : 0,
                      N, H, 1, dk, dv};
    const hipError_t err = glr::launch_vla(dtype == LA_BF16, args, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(LA_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
    return LA_OK;
}

const char* la_status_str(la_status status) {
    switch (status) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID: return "invalid argument";
        case LA_ERR_UNSUPPORTED: return "unsupported shape";
        case LA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

const char* la_last_error(void) { return g_last_error; }

int la_version(void) { return (3 << 16) | 4; }

}  // extern "C"
