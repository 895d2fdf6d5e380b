// bf16 backward of the gated delta rule, chunk 16: instantiation (kernels in chunk_delta_bwd.hpp).
#include "chunk_delta_bwd.hpp"

namespace glr {
hipError_t launch_chunk_bwd_gdelta_c16(const BwdArgs& a, hipStream_t stream) {
    return ck::launch_gdelta_bwd<16>(a, stream);
}
}  // namespace glr
