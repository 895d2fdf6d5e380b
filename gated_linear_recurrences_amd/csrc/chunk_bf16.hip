// Dispatch of the bf16 MFMA chunk kernels by gate variant.
#include "launch.hpp"

namespace glr {

hipError_t launch_chunk_bf16_retention(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gla(const ChunkArgs& a, hipStream_t stream);
hipError_t launch_chunk_bf16_gdelta(const ChunkArgs& a, hipStream_t stream);

hipError_t launch_chunk_bf16(Variant variant, const ChunkArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    switch (variant) {
        case kRetention: return launch_chunk_bf16_retention(a, stream);
        case kGLA: return launch_chunk_bf16_gla(a, stream);
        case kGDelta: return launch_chunk_bf16_gdelta(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace glr
