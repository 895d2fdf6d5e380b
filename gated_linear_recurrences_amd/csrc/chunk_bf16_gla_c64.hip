// bf16 chunked forward, gla, chunk 64: instantiation of the single pass (chunk_gla_sp.hpp, d_k
// >= 32 with enough sequences) and the two-pass kernels (chunk_state.hpp, chunk_output.hpp).
#include "chunk_gla_sp.hpp"
#include "chunk_two_pass.hpp"

namespace glr {
hipError_t launch_chunk_bf16_gla_c64(const ChunkArgs& a, hipStream_t stream) {
    if (gla_single_pass(a)) return ck::launch_gla_sp(a, stream);
    return ck::launch_two_pass<64, ck::kGateChannel>(a, stream);
}
}  // namespace glr
