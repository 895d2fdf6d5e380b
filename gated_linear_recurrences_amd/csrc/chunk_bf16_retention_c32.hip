// bf16 chunked forward, retention, chunk 32: instantiation of the single-pass kernel
// (chunk_fused.hpp) and the two-pass kernels (chunk_state.hpp, chunk_output.hpp).
#include "chunk_fused.hpp"
#include "chunk_two_pass.hpp"

namespace glr {
hipError_t launch_chunk_bf16_retention_c32(const ChunkArgs& a, hipStream_t stream) {
    if (single_pass_forward(kRetention, a)) return ck::launch_fused<32, ck::kGateFixed>(a, stream);
    return ck::launch_two_pass<32, ck::kGateFixed>(a, stream);
}
}  // namespace glr
