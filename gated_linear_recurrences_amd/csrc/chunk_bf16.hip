// Dispatch of the bf16 MFMA chunk kernels by gate variant and chunk length.
#include "chunk_delta_sp.hpp"
#include "launch.hpp"

namespace glr {

hipError_t launch_chunk_bf16_retention_c16(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_retention_c32(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_retention_c64(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gla_c16(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gla_c32(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gla_c64(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_scalar_c16(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_scalar_c32(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_scalar_c64(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gdelta_c16(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gdelta_c32(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gdelta_c64(const ChunkArgs& a, hipStream_t stream);

size_t chunk_workspace_bytes(Variant variant, const ChunkArgs& a, bool bf16) {
    if (!bf16 || a.B == 0 || a.H == 0) return 0;
    const size_t chunks = static_cast<size_t>((a.T + a.chunk - 1) / a.chunk);
    if (single_pass_forward(variant, a)) return 0;
    if (variant == kGLA && gla_single_pass(a)) return 0;
    if (variant == kGDelta && delta_single_pass(a))
        return ck::dsp_ws_bytes(static_cast<int64_t>(a.B) * a.H * chunks, a.chunk, a.dk, (a.fuse & 1) != 0);
    if (variant == kGDelta)
        return ck::delta_ws_bytes(static_cast<int64_t>(a.B) * a.H * chunks, a.chunk, a.dk, a.dv, (a.fuse & 1) != 0);
    return static_cast<size_t>(a.B) * a.H * chunks * a.dv * a.dk * 2;
}

// Retention's and the scalar decay's output norm (fuse bits 1, 2): a pass over the output
// rows once the chunk kernels are done (their value slices sit in different workgroups).
static hipError_t norm_rows_bf16(hipError_t err, const ChunkArgs& a, hipStream_t stream) {
    if (err != hipSuccess || !(a.fuse & 6)) return err;
    switch (a.dv) {
        case 16: return ck::launch_norm_rows_bf16<16>(a, stream);
        case 32: return ck::launch_norm_rows_bf16<32>(a, stream);
        case 64: return ck::launch_norm_rows_bf16<64>(a, stream);
        case 128: return ck::launch_norm_rows_bf16<128>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_bf16(Variant variant, const ChunkArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    switch (variant) {
        case kRetention:
            if (a.chunk == 16) return norm_rows_bf16(launch_chunk_bf16_retention_c16(a, stream), a, stream);
            if (a.chunk == 32) return norm_rows_bf16(launch_chunk_bf16_retention_c32(a, stream), a, stream);
            if (a.chunk == 64) return norm_rows_bf16(launch_chunk_bf16_retention_c64(a, stream), a, stream);
            break;
        case kScalar:
            if (a.chunk == 16) return norm_rows_bf16(launch_chunk_bf16_scalar_c16(a, stream), a, stream);
            if (a.chunk == 32) return norm_rows_bf16(launch_chunk_bf16_scalar_c32(a, stream), a, stream);
            if (a.chunk == 64) return norm_rows_bf16(launch_chunk_bf16_scalar_c64(a, stream), a, stream);
            break;
        case kGLA:
            if (a.chunk == 16) return launch_chunk_bf16_gla_c16(a, stream);
            if (a.chunk == 32) return launch_chunk_bf16_gla_c32(a, stream);
            // the single pass leaves GLA's layer norm to a pass over the rows (the two-pass
            // output kernel applies it in place)
            if (a.chunk == 64)
                return gla_single_pass(a) ? norm_rows_bf16(launch_chunk_bf16_gla_c64(a, stream), a, stream)
                                          : launch_chunk_bf16_gla_c64(a, stream);
            break;
        case kGDelta:
            if (a.chunk == 16) return launch_chunk_bf16_gdelta_c16(a, stream);
            if (a.chunk == 32) return launch_chunk_bf16_gdelta_c32(a, stream);
            if (a.chunk == 64) return launch_chunk_bf16_gdelta_c64(a, stream);
            break;
    }
    return hipErrorInvalidValue;
}

}  // namespace glr
