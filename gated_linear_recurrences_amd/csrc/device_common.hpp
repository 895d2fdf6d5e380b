// Device-side helpers shared by the gfx950 kernels: storage conversions, MFMA
// wrappers and wavefront reductions / scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- storage types

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
    return __uint_as_float(static_cast<unsigned int>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (NaN kept quiet).
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(unsigned short, h);
}

// Element loads/stores for the two storage types of q, k, v, o.
template <typename TS> struct Store;

template <> struct Store<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float x) { p[i] = x; }
};

template <> struct Store<unsigned short> {
    static __device__ __forceinline__ float load(const unsigned short* p, int64_t i) {
        return bf16_bits_to_f32(p[i]);
    }
    static __device__ __forceinline__ void store(unsigned short* p, int64_t i, float x) {
        p[i] = f32_to_bf16_bits(x);
    }
};

// ---------------------------------------------------------------- MFMA (CDNA4)
//
// v_mfma_f32_16x16x32_bf16: D[16x16] += A[16x32] * B[32x16] per wavefront.
// Lane l (r = l & 15, g = l >> 4) supplies A[r][8g .. 8g+7] and B[8g .. 8g+7][r]
// and holds D[4g .. 4g+3][r].  The eight k-slots of a lane may be any eight
// reduction indices as long as A and B use the same assignment.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3,
                                        float a4, float a5, float a6, float a7) {
    bf16x8 r;
    r[0] = static_cast<__bf16>(a0); r[1] = static_cast<__bf16>(a1);
    r[2] = static_cast<__bf16>(a2); r[3] = static_cast<__bf16>(a3);
    r[4] = static_cast<__bf16>(a4); r[5] = static_cast<__bf16>(a5);
    r[6] = static_cast<__bf16>(a6); r[7] = static_cast<__bf16>(a7);
    return r;
}

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
    return pack8(lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]);
}

__device__ __forceinline__ bf16x8 join8(bf16x4 lo, bf16x4 hi) {
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

// ---------------------------------------------------------------- workgroup barrier

// Barrier for LDS traffic only: waits for this wave's LDS operations, then for
// every wave of the workgroup. Unlike __syncthreads() it does not drain
// outstanding global loads, so a prefetch of the next chunk stays in flight
// across it. Valid only where no other wave reads this wave's global writes.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- wavefront helpers

// Sum over groups of `width` consecutive lanes (width a power of two <= 64);
// every lane of a group receives the group's sum.
template <int width>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = width / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over each row of 16 lanes with DPP moves (no LDS crossbar): quad swaps, then the
// half-row and row mirrors; every lane of the row receives the row's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __uint_as_float(static_cast<unsigned>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(__float_as_uint(x)), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_move<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_move<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_move<0x141>(x);   // row_half_mirror
    x += dpp_move<0x140>(x);   // row_mirror
    return x;
}

// Sum over the four rows of 16 lanes (lanes of equal lane & 15) with the gfx950 row
// swaps: each swap leaves a lane holding its own value and its partner row's.
__device__ __forceinline__ float cross_row_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over all 64 lanes, received by every lane.
__device__ __forceinline__ float wave_sum(float x) { return cross_row_sum(row16_sum(x)); }

// Inclusive prefix sum across the 64 lanes of a wavefront (Hillis-Steele).
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// The same scan with DPP moves and lane reads (no LDS crossbar): a Hillis-Steele scan within
// each row of 16 lanes (row_shr by 1, 2, 4, 8; lanes shifted in from outside the row read 0),
// then each row adds the totals of the rows before it (lanes 15, 31 and 47 read as scalars).
__device__ __forceinline__ float wave_inclusive_scan_dpp(float x) {
    x += dpp_move<0x111>(x);   // row_shr:1
    x += dpp_move<0x112>(x);   // row_shr:2
    x += dpp_move<0x114>(x);   // row_shr:4
    x += dpp_move<0x118>(x);   // row_shr:8
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
}

}  // namespace glr
