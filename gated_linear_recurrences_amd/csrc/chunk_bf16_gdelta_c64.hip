// bf16 three-kernel chunked forward, gated delta rule, chunk 64: instantiation (kernels in chunk_delta.hpp).
#include "chunk_delta.hpp"

namespace glr {
hipError_t launch_chunk_bf16_gdelta_c64(const ChunkArgs& a, hipStream_t stream) {
    return ck::launch_delta<64>(a, stream);
}
}  // namespace glr
