// bf16 two-pass chunked forward, retention, chunk 32: instantiation (kernels in chunk_state.hpp, chunk_output.hpp).
#include "chunk_two_pass.hpp"

namespace glr {
hipError_t launch_chunk_bf16_retention_c32(const ChunkArgs& a, hipStream_t stream) {
    return ck::launch_two_pass<32, ck::kGateFixed>(a, stream);
}
}  // namespace glr
