// bf16 two-pass chunked forward, scalar data-dependent decay, chunk 64: instantiation (kernels in chunk_state.hpp, chunk_output.hpp).
#include "chunk_two_pass.hpp"

namespace glr {
hipError_t launch_chunk_bf16_scalar_c64(const ChunkArgs& a, hipStream_t stream) {
    return ck::launch_two_pass<64, ck::kGateScalar>(a, stream);
}
}  // namespace glr
