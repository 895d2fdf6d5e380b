// bf16 two-pass chunked forward, gla, chunk 16: instantiation (kernels in chunk_state.hpp, chunk_output.hpp).
#include "chunk_two_pass.hpp"

namespace glr {
hipError_t launch_chunk_bf16_gla_c16(const ChunkArgs& a, hipStream_t stream) {
    return ck::launch_two_pass<16, ck::kGateChannel>(a, stream);
}
}  // namespace glr
