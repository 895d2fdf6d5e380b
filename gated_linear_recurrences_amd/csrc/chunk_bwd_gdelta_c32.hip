// bf16 backward of the gated delta rule, chunk 32: instantiation (kernels in chunk_delta_bwd.hpp).
#include "chunk_delta_bwd.hpp"

namespace glr {
hipError_t launch_chunk_bwd_gdelta_c32(const BwdArgs& a, hipStream_t stream) {
    return ck::launch_gdelta_bwd<32>(a, stream);
}
}  // namespace glr
