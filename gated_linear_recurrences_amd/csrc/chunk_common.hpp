// Device helpers shared by the bf16 chunk kernels (gfx950).
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace glr {
namespace ck {

typedef unsigned short u16;
constexpr float kLog2e = 1.4426950408889634f;

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

// Column of the 8-element piece that lane group g supplies in reduction block kb (of KB
// 32-wide blocks) of an MFMA operand read row-wise from a SwzTile. Any one-to-one
// assignment gives the same sum when both operands of the product use it; this one keeps
// the row reads free of LDS bank conflicts on gfx950, where a 16-byte read serves lanes
// 0-7 together with 24-31 (and 8-15 with 16-23): rows 0-7 of group 0 meet rows 8-15 of
// group 1 in one cycle, the 64- and 128-wide swizzles send those two row halves of one
// chunk to chunks of opposite parity, and pieces of equal parity for groups 0/1 (and 2/3)
// then land on distinct banks. Pieces 4kb+g (the plain order) would collide two-way. Padded
// tiles (row stride d + 16) keep the plain order, which is already conflict-free there.
__device__ __forceinline__ int rr_col(int kb, int g, int KB) { return 8 * (kb + KB * g); }

// Split operand over 32 rows (two 16-row halves) read transposed: rows 32jb + [0, 32) of
// column tile n0; the second half zero unless `hi`.
template <int RS>
__device__ __forceinline__ bf16x8 tr_split(const u16* X, int jb, int n0, bool hi, int r16, int g) {
    return join8(tr_op<RS>(X, 32 * jb, n0, r16, g), hi ? tr_op<RS>(X, 32 * jb + 16, n0, r16, g) : zero4());
}

// Row-major LDS tile of W bf16 elements per row. For W = 64 and 128 the rows are
// unpadded and the 16-byte chunks of row r sit permuted by XOR with h(r), chosen so
// that both access patterns of the MFMA operands hit 64 distinct banks: a row read (16
// consecutive rows, one chunk each: h is one-to-one on them) and a transposing read
// (8 consecutive rows, two adjacent chunks each: h / 2 is one-to-one on the rows that
// share a bank line). Narrower tiles keep the padded stride tile_stride(W).
// Reference of a 16-token tile in the per-channel gate factorisation (log2 units): the
// cumulative gate r just before the tile, moved down to at most 80 nats (115.4 in log2
// units) above the gate at the tile's last token, so that e^(G - ref) and e^(ref - G) stay
// within e^(+-80) for every token of any tile whose gates sum to -160 nats or more.
__device__ __forceinline__ float tile_ref(float r, float last) { return fminf(r, last + 115.4f); }
__device__ __forceinline__ f32x4 tile_ref4(f32x4 r, f32x4 last) {
    f32x4 m;
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = tile_ref(r[e], last[e]);
    return m;
}

template <int W>
struct SwzTile {
    static constexpr int STRIDE = (W == 64 || W == 128) ? W : (W == 16 ? 16 : W + 16);
    __device__ static __forceinline__ int off(int r, int c) {
        if constexpr (W == 128) {
            const int h = ((r & 7) << 1) | ((r >> 3) & 1);
            return r * 128 + ((((c >> 3) ^ h) << 3) | (c & 7));
        } else if constexpr (W == 64) {
            const int h = (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
            return r * 64 + ((((c >> 3) ^ h) << 3) | (c & 7));
        } else {
            return r * STRIDE + c;
        }
    }
    // The logical 8-element chunk held at physical chunk p of row r (-1: padding): the
    // inverse of off, for loads that fill a tile in physical order.
    __device__ static __forceinline__ int chunk_at(int r, int p) {
        if constexpr (W == 128) {
            return p ^ (((r & 7) << 1) | ((r >> 3) & 1));
        } else if constexpr (W == 64) {
            return p ^ ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
        } else {
            return p * 8 < W ? p : -1;
        }
    }
};

// tr_op on a SwzTile: lane (r, g) receives X[base+4g+e][n0+r], e = 0..3.
template <int W>
__device__ __forceinline__ bf16x4 tr_op_s(const u16* X, int base, int n0, int r16, int g) {
    const u16* p = X + SwzTile<W>::off(base + 4 * g + (r16 >> 2), n0 + 4 * (r16 & 3));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// ds_read_b64_tr_b16 at a lane's own address: the four 16-bit values a lane reads are
// handed to the four lanes of its column quad, one each (see tr_op_s).
__device__ __forceinline__ bf16x4 tr4(const u16* p) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

template <int W>
__device__ __forceinline__ bf16x8 tr_split_s(const u16* X, int jb, int n0, bool hi, int r16, int g) {
    return join8(tr_op_s<W>(X, 32 * jb, n0, r16, g), hi ? tr_op_s<W>(X, 32 * jb + 16, n0, r16, g) : zero4());
}

// Row stride (bf16 elements) of a staged token-major tile `width` channels wide:
// 16 more than the width (none for 16-wide tiles), so that rows sit 8 x odd banks
// apart and the 8 rows read by half a wave of ds_read_b64_tr_b16 (8 bytes from
// each of 4 lanes per row) fall on distinct banks of the 64.
constexpr int tile_stride(int width) { return width == 16 ? 16 : width + 16; }

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 x) { return __builtin_bit_cast(bf16x8, x); }

// DeltaNet's feature map on a row of q or k held as 16-byte pieces by PPR consecutive
// lanes (a PPR-aligned group): SiLU x / (1 + e^-x) per element, then the row scaled to
// unit L2 norm; the squared sum meets across the group by butterfly shuffles. Every
// lane of the wave must take part (groups are uniformly valid or ignored).
template <int PPR>
__device__ __forceinline__ u16x8 silu_l2_piece(u16x8 raw) {
    float y[8];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = bf16_bits_to_f32(raw[e]);
        y[e] = x * __builtin_amdgcn_rcpf(1.f + ex2(-x * kLog2e));   // ~1 ulp; the result is rounded to bf16
        ss += y[e] * y[e];
    }
#pragma unroll
    for (int off = 1; off < PPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
    u16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = f32_to_bf16_bits(y[e] * inv);
    return out;
}

// Scale four bf16 values by four fp32 factors (round to bf16 again).
__device__ __forceinline__ bf16x4 scale4(bf16x4 x, f32x4 s) { return cvt4(up4(x) * s); }

// Block index -> (head, value tile), XCD-aware: consecutive workgroup ids land on
// different XCDs, so the value tiles of one head get ids that share an XCD and its L2.
__device__ __forceinline__ int logical_block_of(unsigned bid, unsigned grid, int remap) {
    return remap ? static_cast<int>((bid & 7) * (grid >> 3) + (bid >> 3)) : static_cast<int>(bid);
}

}  // namespace ck
}  // namespace glr

namespace glr {
namespace ck {

constexpr int kCUs = 256;   // compute units of an MI355X

// Gate of the chunk kernels: one fixed decay per head, one data-dependent gate per key
// channel, or one data-dependent scalar per token; the gated delta rule's single pass (a
// scalar gate whose cumulative sums come from its prep) is the fourth kind.
enum GateKind { kGateFixed = 0, kGateChannel = 1, kGateScalar = 2, kGateDeltaRule = 3 };

}  // namespace ck
}  // namespace glr
