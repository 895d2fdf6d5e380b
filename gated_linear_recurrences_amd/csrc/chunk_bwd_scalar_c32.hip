// bf16 backward, scalar data-dependent decay, chunk 32: instantiation (kernels in chunk_backward.hpp).
#include "chunk_backward.hpp"

namespace glr {
hipError_t launch_chunk_bwd_scalar_c32(const BwdArgs& a, hipStream_t stream) {
    return ck::launch_backward<32, ck::kGateScalar>(a, stream);
}
}  // namespace glr
