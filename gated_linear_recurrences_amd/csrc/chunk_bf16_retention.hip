// bf16 MFMA chunk kernels, retention instantiations (kernel template in chunk_bf16.hpp).
#include "chunk_bf16.hpp"

namespace glr {
hipError_t launch_chunk_bf16_retention(const ChunkArgs& a, hipStream_t stream) {
    return bf16k::launch_variant<kRetention>(a, stream);
}
}  // namespace glr
