// Internal launch interface between the C ABI (glr_api.cpp) and the kernels.
// Arguments reaching these functions have been validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace glr {

enum Variant { kRetention = 0, kGLA = 1, kGDelta = 2, kScalar = 3 };

// Records `message` as the calling thread's last error and returns `status` (an la_status).
int report_error(int status, const char* message);
struct ChunkArgs;
// The argument checks of a chunk entry point (sizes, dtype, pointers), as an la_status.
int check_chunk_call(Variant variant, const ChunkArgs& a, int dtype);

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* gate;   // retention: log_gamma [H]; GLA: log_alpha [B,H,T,dk]; gdelta, scalar: log_alpha [B,H,T]
    const float* beta;   // gdelta only: [B,H,T]
    const float* s0;     // [B,H,dv,dk] or nullptr
    void* o;             // [B,H,T,dv]
    float* s_out;        // [B,H,dv,dk] or nullptr
    int B, H, T, dk, dv, chunk;
    void* ws;            // device workspace of at least chunk_workspace_bytes() bytes
    // gated delta rule: bit 0 - q, k are mapped by SiLU then L2 normalisation per token on
    // load; bit 1 - each output row is RMS-normalised with weight onw [dv] and eps oeps.
    // GLA: bit 2 - each output row is layer-normalised (mean 0, variance 1 with eps oeps),
    // times onw [dv] plus onb [dv] (onb may be null)
    int fuse;
    const float* onw;
    float oeps;
    const float* onb;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;  // GLA: [N,H,dk]; gated delta: [N,H]
    const float* beta;   // gated delta: [N,H]; nullptr for the GLA step
    float* s;
    void* o;
    int N, H, dk, dv;
};

// Backward of the fixed, scalar or per-channel (GLA) decay and of the gated delta rule (bf16
// storage).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* gate;    // fixed: log_gamma [H]; scalar: log_alpha [B,H,T]; GLA: log_alpha [B,H,T,dk]
    const float* s0;      // [B,H,dv,dk] or nullptr
    const void* dout;     // [B,H,T,dv]: gradient of o
    const float* ds_out;  // [B,H,dv,dk] or nullptr: gradient of the final memory
    void* grad_q;         // [B,H,T,dk]
    void* grad_k;         // [B,H,T,dk]
    void* grad_v;         // [B,H,T,dv]
    float* dgate;         // fixed: [H]; scalar: [B,H,T]; GLA: [B,H,T,dk]
    float* ds0;           // [B,H,dv,dk] or nullptr
    int B, H, T, dk, dv, chunk;
    void* ws;             // device workspace of at least bwd_workspace_size() bytes
    const float* beta;    // gated delta rule: write strengths [B,H,T]
    float* dbeta;         // gated delta rule: their gradient [B,H,T]
};
size_t bwd_workspace_size(Variant variant, const BwdArgs& a);
hipError_t launch_chunk_bwd(Variant variant, const BwdArgs& a, hipStream_t stream);

// Variational linear attention over whole sequences (T = 1 and the memory and penalty
// in place: the decode step).
struct VlaArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* u;        // penalty directions [B,H,T,dk]
    float inv_lambda0;    // A_0 = I * inv_lambda0 when a0 is nullptr
    const float* a0;      // [B,H,dk,dk] or nullptr
    const float* s0;      // [B,H,dv,dk] or nullptr
    const float* n0;      // ratio readout: [B,H,dk] or nullptr (zeros)
    void* o;              // [B,H,T,dv]
    float* s_out;         // [B,H,dv,dk] or nullptr (may equal s0)
    float* a_out;         // [B,H,dk,dk] or nullptr (may equal a0)
    float* n_out;         // ratio readout: [B,H,dk] or nullptr (may equal n0)
    int ratio;            // 1: ELU+1 ratio readout; 0: o = S q
    int B, H, T, dk, dv;
};
hipError_t launch_vla(bool bf16, const VlaArgs& a, hipStream_t stream);

// Retention and the scalar decay (bf16 storage) take the single-pass forward, which needs no
// workspace, when the sequences times the 16-channel value slices fill at least half the
// CUs; with fewer, the two-pass form spreads the chunks of each sequence over the chip.
inline bool single_pass_forward(Variant variant, const ChunkArgs& a) {
    return (variant == kRetention || variant == kScalar) &&
           static_cast<long long>(a.B) * a.H * (a.dv / 16) >= 128;
}

// GLA (bf16 storage) at chunk 64 with d_k of 64 or 128 takes its single pass (no workspace) under the
// same occupancy rule as retention; its buffer offsets are 31-bit (one sequence's raw gates,
// rows padded to whole chunks, below 2^31 bytes: T below 2^22 tokens at d_k = 128).
inline bool gla_single_pass(const ChunkArgs& a) {
    const long long rows = (static_cast<long long>(a.T) + 63) / 64 * 64;
    const long long per_row = a.dk * 4 > a.dv * 2 ? a.dk * 4 : a.dv * 2;
    return a.chunk == 64 && a.dk >= 64 && static_cast<long long>(a.B) * a.H * (a.dv / 16) >= 128 &&
           rows * per_row < (1ll << 31);
}

// The gated delta rule (bf16 storage) at chunk 64 with d_k >= 32 takes the prep + single-pass
// form (T_U and the gates per chunk in the workspace, the mapped q and k too when the feature
// map is fused in); chunks of 16 and 32 and d_k = 16 take the three-kernel form.
// (Its buffer offsets are 31-bit: one sequence's q, k, v or o, and its T_U, must stay below
// 2^31 bytes, which holds for T below 2^22 tokens at d = 128.)
inline bool delta_single_pass(const ChunkArgs& a) {
    const long long rows = (static_cast<long long>(a.T) + 63) / 64 * 64;
    const long long d = a.dk > a.dv ? a.dk : a.dv;
    return a.chunk == 64 && a.dk >= 32 && rows * (d > 64 ? d : 64) * 2 < (1ll << 31);
}

// Retention and the scalar decay (bf16 storage) at chunk 64 with d_k >= 32 take the gated
// delta rule's single pass without its delta step (same 31-bit buffer offsets).
inline bool linear_single_pass(const ChunkArgs& a) {
    const long long rows = (static_cast<long long>(a.T) + 63) / 64 * 64;
    const long long d = a.dk > a.dv ? a.dk : a.dv;
    return a.chunk == 64 && a.dk >= 32 && rows * (d > 64 ? d : 64) * 2 < (1ll << 31);
}

// float32 storage, fp32 arithmetic (VALU).
hipError_t launch_chunk_f32(Variant variant, const ChunkArgs& a, hipStream_t stream);
// Device workspace the chunk kernels of (variant, shape, storage) need, in bytes.
size_t chunk_workspace_bytes(Variant variant, const ChunkArgs& a, bool bf16);
// bfloat16 storage, bf16 MFMA with fp32 accumulation and fp32 memory.
hipError_t launch_chunk_bf16(Variant variant, const ChunkArgs& a, hipStream_t stream);
// one decode token (the gated delta rule when a.beta is set); bf16 == true for
// bfloat16 token storage.
hipError_t launch_decode(bool bf16, const DecodeArgs& a, hipStream_t stream);

}  // namespace glr
