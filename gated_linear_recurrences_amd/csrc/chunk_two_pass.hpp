// Launch of the two-pass chunked forward (state pass, then output pass) for
// retention, the scalar data-dependent decay and GLA with bf16 storage. The memory entering each chunk travels
// between the passes through the caller's workspace, [B*H][chunks][d_v][d_k] bf16.
#pragma once

#include "chunk_output.hpp"
#include "chunk_state.hpp"

namespace glr {
namespace ck {

// State-pass workgroup: NW = min(4, d_k / 16) key tiles of 16 channels against
// DVB = 16 TV value channels (two waves per key tile when TV >= 2): the widest value block (fewest re-reads of
// k and the gates) that still gives each CU a workgroup, TV = 1 when even the
// narrowest cannot.
constexpr int state_key_tiles(int dk) { return dk / 16 < 4 ? dk / 16 : 4; }

inline int state_value_tiles(int64_t heads, int dv, int dk) {
    const int kblocks = dk / (16 * state_key_tiles(dk));
    for (int tv = 8; tv >= 1; tv >>= 1)
        if (16 * tv <= dv && heads * (dv / (16 * tv)) * kblocks >= kCUs) return tv;
    return 1;
}

// Bytes per lane of one slot of the state pass's register ring: U chunks of k, v (and
// GLA's fp32 gates) over the workgroup's 64 NW lanes.
template <int C, int NW, int TV, int GK>
constexpr int state_ring_bytes(int U) {
    return U * C * (16 * NW * 2 + 16 * TV * 2 + (GK == kGateChannel ? 16 * NW * 4 : 0)) / (64 * NW);
}

// chunks per workgroup barrier: the largest of 4, 2, 1 whose double-buffered staging fits
// in LDS and whose ring slot stays within 384 bytes per lane (with d_k = 16 a single wave
// would otherwise hold four chunks of 128 value channels per slot, 1152 bytes, and spill)
template <int C, int NW, int TV, int GK>
constexpr int state_group() {
    constexpr int kRing = 384;
    return (StateLayout<C, NW, TV, 4, GK>::fits && state_ring_bytes<C, NW, TV, GK>(4) <= kRing) ? 4
           : (StateLayout<C, NW, TV, 2, GK>::fits && state_ring_bytes<C, NW, TV, GK>(2) <= kRing) ? 2
                                                                                                   : 1;
}

template <int C, int DK, int TV, int GK, bool REV = false>
hipError_t launch_state(const ChunkArgs& a, int NC, hipStream_t stream) {
    constexpr int NW = state_key_tiles(DK);
    // one wave per key tile holding all TV value tiles: the key operand (and, for GLA, the
    // per-chunk gate scan) is then read once per key tile; two waves per key tile sharing the
    // value tiles measured 12% slower for GLA B8 H16 T4096 and no faster for retention
    constexpr int NWV = 1;
    constexpr int U = state_group<C, NW, TV, GK>();
    StateParams p{};
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.gate = a.gate;
    p.s0 = a.s0;
    p.states = static_cast<u16*>(a.ws);
    p.s_out = a.s_out;
    p.H = a.H;
    p.T = a.T;
    p.dv = a.dv;
    p.NC = NC;
    p.vblocks = a.dv / (16 * TV);
    p.kblocks = DK / (16 * NW);
    const int64_t G = static_cast<int64_t>(a.B) * a.H * p.vblocks * p.kblocks;
    p.remap = (G % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((state_kernel<C, DK, NW, NWV, TV, U, GK, REV>), dim3(static_cast<unsigned>(G)), dim3(64 * NW * NWV),
                       0, stream, p);
    return hipGetLastError();
}

template <int C, int DK, int DV, int GK>
hipError_t launch_two_pass_dv(const ChunkArgs& a, hipStream_t stream) {
    const int NC = (a.T + C - 1) / C;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    hipError_t err = hipErrorInvalidValue;
    switch (state_value_tiles(heads, DV, DK)) {
        case 8: if constexpr (DV >= 128) err = launch_state<C, DK, 8, GK>(a, NC, stream); break;
        case 4: if constexpr (DV >= 64) err = launch_state<C, DK, 4, GK>(a, NC, stream); break;
        case 2: if constexpr (DV >= 32) err = launch_state<C, DK, 2, GK>(a, NC, stream); break;
        default: err = launch_state<C, DK, 1, GK>(a, NC, stream); break;
    }
    if (err != hipSuccess || NC == 0) return err;
    OutParams p{};
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.gate = a.gate;
    p.states = static_cast<const u16*>(a.ws);
    p.o = static_cast<u16*>(a.o);
    p.H = a.H;
    p.T = a.T;
    p.NC = NC;
    p.lnw = (a.fuse & 4) ? a.onw : nullptr;
    p.lnb = (a.fuse & 4) ? a.onb : nullptr;
    p.lneps = a.oeps;
    // four waves for the scalar gates (two or three workgroups per CU), eight for GLA,
    // whose larger LDS footprint allows two workgroups per CU
    constexpr int NW = GK == kGateChannel ? 8 : 4;
    hipLaunchKernelGGL((output_kernel<C, DK, DV, GK, NW>), dim3(static_cast<unsigned>(heads * NC)), dim3(64 * NW),
                       0, stream, p);
    return hipGetLastError();
}

template <int C, int DK, int GK>
hipError_t launch_two_pass_dk(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_two_pass_dv<C, DK, 16, GK>(a, stream);
        case 32: return launch_two_pass_dv<C, DK, 32, GK>(a, stream);
        case 64: return launch_two_pass_dv<C, DK, 64, GK>(a, stream);
        case 128: return launch_two_pass_dv<C, DK, 128, GK>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int C, int GK>
hipError_t launch_two_pass(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_two_pass_dk<C, 16, GK>(a, stream);
        case 32: return launch_two_pass_dk<C, 32, GK>(a, stream);
        case 64: return launch_two_pass_dk<C, 64, GK>(a, stream);
        case 128: return launch_two_pass_dk<C, 128, GK>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
