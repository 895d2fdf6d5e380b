// bf16 backward, gate per key channel (GLA), chunk 32: instantiation (kernels in chunk_backward_gla.hpp).
#include "chunk_backward_gla.hpp"

namespace glr {
hipError_t launch_chunk_bwd_gla_c32(const BwdArgs& a, hipStream_t stream) {
    return ck::launch_backward_gla<32>(a, stream);
}
}  // namespace glr
