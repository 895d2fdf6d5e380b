// bf16 chunked forward, scalar data-dependent decay, chunk 64: instantiation of the single-pass
// kernels (chunk_delta_sp.hpp at d_k >= 32, chunk_fused.hpp at d_k = 16) and the two-pass
// kernels (chunk_state.hpp, chunk_output.hpp).
#include "chunk_delta_sp.hpp"
#include "chunk_fused.hpp"
#include "chunk_two_pass.hpp"

namespace glr {
hipError_t launch_chunk_bf16_scalar_c64(const ChunkArgs& a, hipStream_t stream) {
    if (single_pass_forward(kScalar, a))
        return linear_single_pass(a) ? ck::launch_lsp<64, ck::kGateScalar>(a, stream) : ck::launch_fused<64, ck::kGateScalar>(a, stream);
    return ck::launch_two_pass<64, ck::kGateScalar>(a, stream);
}
}  // namespace glr
