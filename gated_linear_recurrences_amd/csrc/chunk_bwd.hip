// Dispatch of the bf16 backward kernels by gate variant and chunk length.
#include "chunk_backward_gla.hpp"
#include "chunk_delta_bwd.hpp"
#include "launch.hpp"

namespace glr {

hipError_t launch_chunk_bwd_retention_c16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_retention_c32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_retention_c64(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_scalar_c16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_scalar_c32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_scalar_c64(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_gla_c16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_gla_c32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_gla_c64(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_gdelta_c16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_gdelta_c32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_chunk_bwd_gdelta_c64(const BwdArgs& a, hipStream_t stream);

size_t bwd_workspace_size(Variant variant, const BwdArgs& a) {
    if (a.B == 0 || a.H == 0) return 0;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if (variant == kGLA) return ck::bwd_gla_workspace_bytes(heads, a.T, a.chunk, a.dk, a.dv);
    if (variant == kGDelta) return ck::gd_bwd_ws_bytes(heads * ((static_cast<int64_t>(a.T) + a.chunk - 1) / a.chunk),
                                                       a.chunk, a.dk, a.dv);
    return ck::bwd_workspace_bytes(heads, a.T, a.chunk, a.dk, a.dv);
}

hipError_t launch_chunk_bwd(Variant variant, const BwdArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    if (variant == kRetention) {
        if (a.chunk == 16) return launch_chunk_bwd_retention_c16(a, stream);
        if (a.chunk == 32) return launch_chunk_bwd_retention_c32(a, stream);
        if (a.chunk == 64) return launch_chunk_bwd_retention_c64(a, stream);
    } else if (variant == kScalar) {
        if (a.chunk == 16) return launch_chunk_bwd_scalar_c16(a, stream);
        if (a.chunk == 32) return launch_chunk_bwd_scalar_c32(a, stream);
        if (a.chunk == 64) return launch_chunk_bwd_scalar_c64(a, stream);
    } else if (variant == kGLA) {
        if (a.chunk == 16) return launch_chunk_bwd_gla_c16(a, stream);
        if (a.chunk == 32) return launch_chunk_bwd_gla_c32(a, stream);
        if (a.chunk == 64) return launch_chunk_bwd_gla_c64(a, stream);
    } else if (variant == kGDelta) {
        if (a.chunk == 16) return launch_chunk_bwd_gdelta_c16(a, stream);
        if (a.chunk == 32) return launch_chunk_bwd_gdelta_c32(a, stream);
        if (a.chunk == 64) return launch_chunk_bwd_gdelta_c64(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace glr
