// bf16 three-kernel chunked forward, gated delta rule, chunk 16: instantiation (kernels in chunk_delta.hpp).
#include "chunk_delta.hpp"

namespace glr {
hipError_t launch_chunk_bf16_gdelta_c16(const ChunkArgs& a, hipStream_t stream) {
    return ck::launch_delta<16>(a, stream);
}
}  // namespace glr
