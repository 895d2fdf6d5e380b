// Device helpers shared by the bf16 chunk kernels (gfx950).
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace glr {
namespace ck {

typedef unsigned short u16;
constexpr float kLog2e = 1.4426950408889634f;

struct Params {
    const u16* q;
    const u16* k;
    const u16* v;
    const float* gate;
    const float* beta;
    const float* s0;
    u16* o;
    float* s_out;
    int H, T, dv, tiles, remap;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x4 zero4() {
    const __bf16 z = static_cast<__bf16>(0.f);
    bf16x4 r;
    r[0] = z; r[1] = z; r[2] = z; r[3] = z;
    return r;
}

__device__ __forceinline__ bf16x4 ld4(const u16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ void st4(u16* p, bf16x4 x) { *reinterpret_cast<bf16x4*>(p) = x; }
__device__ __forceinline__ f32x4 ldf4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void stf4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }

__device__ __forceinline__ bf16x4 cvt4(f32x4 x) {
    bf16x4 r;
    r[0] = static_cast<__bf16>(x[0]); r[1] = static_cast<__bf16>(x[1]);
    r[2] = static_cast<__bf16>(x[2]); r[3] = static_cast<__bf16>(x[3]);
    return r;
}

__device__ __forceinline__ f32x4 up4(bf16x4 x) {
    f32x4 r;
    r[0] = static_cast<float>(x[0]); r[1] = static_cast<float>(x[1]);
    r[2] = static_cast<float>(x[2]); r[3] = static_cast<float>(x[3]);
    return r;
}

__device__ __forceinline__ f32x4 zf4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

__device__ __forceinline__ f32x4 mfma16k(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u16 bits(__bf16 x) { return __builtin_bit_cast(u16, x); }

// Vector of N bf16 storage words (N = 4 or 8): the width of one staging load.
template <int N> struct Vec;
template <> struct Vec<8> { typedef u16x8 type; };
template <> struct Vec<4> { typedef u16x4 type; };

// Operand from a row-major LDS array X (row stride RS elements) for reduction block kb
// (MFMA k-slots: lane (r, g) takes columns 32kb + 4g..+3 and 32kb + 16 + 4g..+3 of row
// `row`); the second half is zero when the reduction has only 2*kb+1 tiles.
template <int NTILE, int RS>
__device__ __forceinline__ bf16x8 split_op(const u16* X, int row, int kb, int g) {
    const u16* p = X + row * RS + 32 * kb + 4 * g;
    return join8(ld4(p), (2 * kb + 1 < NTILE) ? ld4(p + 16) : zero4());
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane
// 4a+b receives element b of the 8-byte chunks addressed by lanes a, 4+a, 8+a,
// 12+a. tr_op points lane (r, g) at row base + 4g + r/4, columns n0 + 4(r%4) of a
// row-major array X (row stride RS), so lane (r, g) receives X[base+4g+e][n0+r],
// e = 0..3: four consecutive rows of one column, the MFMA operand layout for a
// reduction over rows.
template <int RS>
__device__ __forceinline__ bf16x4 tr_op(const u16* X, int base, int n0, int r16, int g) {
    const u16* p = X + (base + 4 * g + (r16 >> 2)) * RS + n0 + 4 * (r16 & 3);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// Split operand over 32 rows (two 16-row halves) read transposed: rows 32jb + [0, 32) of
// column tile n0; the second half zero unless `hi`.
template <int RS>
__device__ __forceinline__ bf16x8 tr_split(const u16* X, int jb, int n0, bool hi, int r16, int g) {
    return join8(tr_op<RS>(X, 32 * jb, n0, r16, g), hi ? tr_op<RS>(X, 32 * jb + 16, n0, r16, g) : zero4());
}

// Scale four bf16 values by four fp32 factors (round to bf16 again).
__device__ __forceinline__ bf16x4 scale4(bf16x4 x, f32x4 s) { return cvt4(up4(x) * s); }

// Block index -> (head, value tile), XCD-aware: consecutive workgroup ids land on
// different XCDs, so the value tiles of one head get ids that share an XCD and its L2.
__device__ __forceinline__ int logical_block(const Params& p) {
    int L = blockIdx.x;
    if (p.remap) L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    return L;
}

// Pair index pr (0 .. CT(CT+1)/2 - 1, row order) -> tile pair (it, jt), jt <= it.
__device__ __forceinline__ void pair_of(int pr, int& it, int& jt) {
    it = 0;
    jt = pr;
    while (jt > it) { jt -= it + 1; ++it; }
}

}  // namespace ck
}  // namespace glr

namespace glr {
namespace ck {

// Workgroup shape: the widest value-channel tile (16 * MT, MT in {4, 2, 1}) that
// still gives each of the 256 CUs a workgroup; the key dimension is then split over
// KS = min(d_k / 16, 8 / MT) waves per value tile (up to 8 waves, two per SIMD).
constexpr int kCUs = 256;

inline int choose_mt(int64_t heads, int dv) {
    for (int cand = 4; cand >= 1; cand >>= 1)
        if (16 * cand <= dv && heads * (dv / (16 * cand)) >= kCUs) return cand;
    return 1;
}

template <int DK, int MT>
constexpr int key_split() {
    return (DK / 16 < 8 / MT) ? DK / 16 : 8 / MT;
}

}  // namespace ck
}  // namespace glr
