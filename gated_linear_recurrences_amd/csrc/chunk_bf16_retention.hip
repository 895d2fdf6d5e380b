// bf16 retention chunk kernels: instantiation and launch-shape dispatch (kernel in chunk_ret.hpp).
#include "chunk_ret.hpp"

namespace glr {

namespace {

template <int C, int DK>
hipError_t ret_dk(const ChunkArgs& a, hipStream_t stream) {
    switch (ck::choose_mt(static_cast<int64_t>(a.B) * a.H, a.dv)) {
        case 4: return ck::launch_retention_cfg<C, DK, 4, ck::key_split<DK, 4>()>(a, stream);
        case 2: return ck::launch_retention_cfg<C, DK, 2, ck::key_split<DK, 2>()>(a, stream);
        default: return ck::launch_retention_cfg<C, DK, 1, ck::key_split<DK, 1>()>(a, stream);
    }
}

template <int C>
hipError_t ret_c(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return ret_dk<C, 16>(a, stream);
        case 32: return ret_dk<C, 32>(a, stream);
        case 64: return ret_dk<C, 64>(a, stream);
        case 128: return ret_dk<C, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_bf16_retention(const ChunkArgs& a, hipStream_t stream) {
    switch (a.chunk) {
        case 16: return ret_c<16>(a, stream);
        case 32: return ret_c<32>(a, stream);
        case 64: return ret_c<64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace glr
