// bf16 chunked forward, gated delta rule, chunk 64: instantiation (prep + single pass in
// chunk_delta_sp.hpp; the three-kernel form of chunk_delta.hpp for d_k = 16 and the fused
// entry point).
#include "chunk_delta_sp.hpp"

namespace glr {
hipError_t launch_chunk_bf16_gdelta_c64(const ChunkArgs& a, hipStream_t stream) {
    if (delta_single_pass(a)) return ck::launch_dsp<64>(a, stream);
    return ck::launch_delta<64>(a, stream);
}
}  // namespace glr
