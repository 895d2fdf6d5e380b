// bf16 backward, retention, chunk 64: instantiation (kernels in chunk_backward.hpp).
#include "chunk_backward.hpp"

namespace glr {
hipError_t launch_chunk_bwd_retention_c64(const BwdArgs& a, hipStream_t stream) {
    return ck::launch_backward<64, ck::kGateFixed>(a, stream);
}
}  // namespace glr
