// bf16 MFMA chunk kernels, gdelta instantiations (kernel template in chunk_bf16.hpp).
#include "chunk_bf16.hpp"

namespace glr {
hipError_t launch_chunk_bf16_gdelta(const ChunkArgs& a, hipStream_t stream) {
    return bf16k::launch_variant<kGDelta>(a, stream);
}
}  // namespace glr
