// Variational linear attention ("Riepilogo Tecnico: Attenzione Lineare Variazionale
// (VLA)", sections 2.1-2.3): per token, with the inverse penalty A = M^-1 (d_k x d_k)
// beside the memory S (d_v x d_k),
//   z = A u,  A <- A - z z^T / (1 + u.z)     Sherman-Morrison for M <- M + u u^T
//   a = A k^ / |A k^|,  k^ = k / |k|          normalised gating vector (updated A)
//   S <- S + (v - S k^) a^T                   residual write
// and the readout after the write: the page's ratio of recurrences with the ELU+1
// feature map phi on keys and queries (k^ = phi(k)/|phi(k)|; n, the denominator vector,
// follows the same write driven by the value 1: n <- n + (1 - n.k^) a;
// o = S phi(q) / (n . phi(q))), or o = S q with the key only normalised.
//
// The update is sequential and O(d^2) per token with no dense contraction in it (every
// product is a matrix times one vector), so it runs on the VALU in fp32, all tokens of
// a sequence in one launch: one workgroup per (sequence, head) keeps A and S in
// registers for the whole sequence (or two workgroups, each with half of the rows of S
// and its own copy of the penalty chain, when the sequences are fewer than the CUs).
// Waves 0 .. d_k/16-1 own 16 rows of A each, the other waves 16 rows of S each; lane (r = lane & 15, g = lane >> 4) holds row
// 16w + r, key columns [g d_k/4, (g+1) d_k/4), so a row's dot products meet across
// the four lanes of equal r with two shuffles.
//
// Per token t (one workgroup barrier):
//   A waves, before the barrier: (A u)_m and (A k)_m for their rows, to LDS;
//   barrier;
//   A waves: |k|^2, u.z and z.k^ over the whole vectors (two columns per lane and a
//   wave-wide sum: the same in every wave), A_t k^ and its norm the same way, the
//   rank-1 update of their rows; wave 0 publishes a_t and, for the ratio readout,
//   updates the denominator vector n (two columns per lane) and publishes n_t.phi(q_t);
//   S waves, one token behind: token t-1 with a_{t-1} (published by this barrier).
// LDS vectors are double-buffered by token parity, so no second barrier is needed.
// q, k, u, v are staged through LDS as fp32 in blocks of 16 tokens, two blocks deep:
// each thread loads one 16-byte piece of block b+1 at the start of block b and writes it
// to LDS eight tokens later, so the load latency hides behind eight tokens of work. For
// the ratio readout q and k pass through phi as they are staged.
// Sums over a row's four lane groups use the gfx950 row swaps (v_permlane16/32_swap),
// sums over a row of 16 lanes DPP moves: no LDS crossbar round trips.
//
// One token with the memory and the penalty updated in place (the decode step) is the
// same kernel with T = 1.
#include "device_common.hpp"
#include "launch.hpp"

namespace glr {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kVlaBlock = 16;   // tokens per staged block

template <typename TS, int DK, int DV, int SPL>
struct VlaShape {
    static constexpr int NA = DK / 16;                 // waves holding A
    static constexpr int NS = DV / 16 / SPL;           // waves holding this workgroup's rows of S
    static constexpr int NT = 64 * (NA + NS);
    static constexpr int NCOL = DK / 4;                // key columns per lane
    static constexpr int EPP = 16 / static_cast<int>(sizeof(TS));   // elements per 16-byte piece
    static constexpr int PK = kVlaBlock * DK / EPP;    // pieces of one block of q, k or u
    static constexpr int PV = kVlaBlock * DV / EPP;    // pieces of one block of v
    static constexpr int PTOT = 3 * PK + PV;
    static constexpr int PER = (PTOT + NT - 1) / NT;   // pieces per thread
    static constexpr int SLOT = kVlaBlock * (3 * DK + DV);   // elements of one staged block
};

template <typename TS, int DK, int DV, int SPL>
__global__ __launch_bounds__((VlaShape<TS, DK, DV, SPL>::NT))
void vla_kernel(const TS* __restrict__ q, const TS* __restrict__ k, const TS* __restrict__ v,
                const TS* __restrict__ u, float inv_lambda0, const float* a0, const float* s0,
                const float* n0, TS* __restrict__ o, float* s_out, float* a_out, float* n_out, int ratio,
                int T) {
    using Sh = VlaShape<TS, DK, DV, SPL>;
    constexpr int TB = kVlaBlock, NCOL = Sh::NCOL, NQ = NCOL / 4, NT = Sh::NT;
    constexpr int NC64 = (DK + 63) / 64;                               // columns per lane, whole-vector sums
    constexpr int OK = TB * DK, OU = 2 * TB * DK, OV = 3 * TB * DK;   // offsets in a staged block
    __shared__ __align__(16) float sblk[2][Sh::SLOT];
    __shared__ __align__(16) float sz[2][DK];   // z = A_{t-1} u
    __shared__ __align__(16) float sy[2][DK];   // A_{t-1} k (k not normalised)
    __shared__ __align__(16) float sa[2][DK];   // gating vector a_t
    __shared__ float srk[2];                    // 1 / |k_t|
    __shared__ float sden[2];                   // ratio readout: n_t . phi(q_t)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int c0 = g * NCOL;
    const bool is_a = wave < Sh::NA;
    // SPL workgroups per sequence split the rows of S; each runs the whole penalty chain
    const int part = static_cast<int>(blockIdx.x % SPL);
    const int m = is_a ? 16 * wave + r16 : part * (DV / SPL) + 16 * (wave - Sh::NA) + r16;   // row of A or of S
    const int64_t bh = blockIdx.x / SPL;
    const TS* qg = q + bh * T * DK;
    const TS* kg = k + bh * T * DK;
    const TS* ug = u + bh * T * DK;
    const TS* vg = v + bh * T * DV;
    TS* og = o + bh * T * DV;

    // ---- this lane's slice of A (identity / lambda0 unless handed over) or of S
    float x[NCOL];
    {
        const float* src = is_a ? (a0 ? a0 + (bh * DK + m) * DK + c0 : nullptr)
                                : (s0 ? s0 + (bh * DV + m) * DK + c0 : nullptr);
        if (src) {
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const f32x4 w = *reinterpret_cast<const f32x4*>(src + 4 * i);
                x[4 * i] = w[0]; x[4 * i + 1] = w[1]; x[4 * i + 2] = w[2]; x[4 * i + 3] = w[3];
            }
        } else {
#pragma unroll
            for (int c = 0; c < NCOL; ++c) x[c] = (is_a && m == c0 + c) ? inv_lambda0 : 0.f;
        }
    }

    // ---- ratio readout: wave 0 keeps the denominator vector n, columns lane + 64 i
    float nv[NC64];
#pragma unroll
    for (int i = 0; i < NC64; ++i) {
        const int c = lane + 64 * i;
        nv[i] = (ratio && wave == 0 && n0 != nullptr && (DK % 64 == 0 || c < DK)) ? n0[bh * DK + c] : 0.f;
    }

    // ---- token blocks: piece p of a block is q, k, u or v by range, at element p * EPP of
    // the staged block; tokens past the end read the sequence's first piece (never used)
    u32x4 pend[Sh::PER];
    auto fetch_block = [&](int blk) {
        const int t0 = blk * TB;
#pragma unroll
        for (int i = 0; i < Sh::PER; ++i) {
            int p = tid + i * NT;
            if (Sh::PTOT % NT != 0 && p >= Sh::PTOT) p = 0;
            const TS* src;
            int d, e;
            if (p < Sh::PK) { src = qg; d = DK; e = p * Sh::EPP; }
            else if (p < 2 * Sh::PK) { src = kg; d = DK; e = (p - Sh::PK) * Sh::EPP; }
            else if (p < 3 * Sh::PK) { src = ug; d = DK; e = (p - 2 * Sh::PK) * Sh::EPP; }
            else { src = vg; d = DV; e = (p - 3 * Sh::PK) * Sh::EPP; }
            const int j = e / d;
            const int64_t off = (t0 + j < T) ? static_cast<int64_t>(t0) * d + e : 0;
            pend[i] = *reinterpret_cast<const u32x4*>(src + off);
        }
    };
    // phi = ELU + 1: x + 1 above zero, e^x below
    auto phi4 = [](f32x4 x) {
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = x[e] > 0.f ? x[e] + 1.f : __builtin_amdgcn_exp2f(x[e] * 1.4426950408889634f);
        return y;
    };
    auto stage_block = [&](int slot) {
#pragma unroll
        for (int i = 0; i < Sh::PER; ++i) {
            const int p = tid + i * NT;
            if (Sh::PTOT % NT == 0 || p < Sh::PTOT) {
                float* dst = &sblk[slot][p * Sh::EPP];
                const u32x4 r = pend[i];
                const bool map = ratio && p < 2 * Sh::PK;   // q and k pieces
                if constexpr (sizeof(TS) == 2) {
                    // bf16 pairs: the low half of each word is the earlier element
                    f32x4 lo = f32x4{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u),
                                     __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xffff0000u)};
                    f32x4 hi = f32x4{__uint_as_float(r[2] << 16), __uint_as_float(r[2] & 0xffff0000u),
                                     __uint_as_float(r[3] << 16), __uint_as_float(r[3] & 0xffff0000u)};
                    if (map) {
                        lo = phi4(lo);
                        hi = phi4(hi);
                    }
                    *reinterpret_cast<f32x4*>(dst) = lo;
                    *reinterpret_cast<f32x4*>(dst + 4) = hi;
                } else {
                    f32x4 x = __builtin_bit_cast(f32x4, r);
                    if (map) x = phi4(x);
                    *reinterpret_cast<f32x4*>(dst) = x;
                }
            }
        }
    };

    if (T > 0) {
        fetch_block(0);
        stage_block(0);
    }
    lds_barrier();

    for (int t = 0; t <= T; ++t) {
        // block b + 1 is requested at the first token of block b and staged at its ninth
        if ((t & (TB - 1)) == 0 && t + TB < T) fetch_block(t / TB + 1);
        if ((t & (TB - 1)) == TB / 2 && t + TB / 2 < T) stage_block((t / TB + 1) & 1);
        const int par = t & 1;
        float zm = 0.f;
        if (is_a && t < T) {
            const float* blk = sblk[(t / TB) & 1];
            const int j = t & (TB - 1);
            const float* kr = blk + OK + j * DK + c0;
            const float* ur = blk + OU + j * DK + c0;
            float zp = 0.f, yp = 0.f;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const f32x4 kk = *reinterpret_cast<const f32x4*>(kr + 4 * i);
                const f32x4 uu = *reinterpret_cast<const f32x4*>(ur + 4 * i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zp += x[4 * i + e] * uu[e];
                    yp += x[4 * i + e] * kk[e];
                }
            }
            zm = cross_row_sum(zp);
            yp = cross_row_sum(yp);
            if (g == 0) {
                sz[par][m] = zm;
                sy[par][m] = yp;
            }
        }
        lds_barrier();
        if (is_a) {
            if (t < T) {
                const float* blk = sblk[(t / TB) & 1];
                const int j = t & (TB - 1);
                // whole-vector sums: columns lane, lane + 64
                float zc[NC64], yc[NC64], kcol[NC64];
                float kn = 0.f, uz = 0.f, zkr = 0.f;
#pragma unroll
                for (int i = 0; i < NC64; ++i) {
                    const int c = lane + 64 * i;
                    zc[i] = yc[i] = kcol[i] = 0.f;
                    if (DK % 64 == 0 || c < DK) {
                        const float kc = blk[OK + j * DK + c], uc = blk[OU + j * DK + c];
                        kcol[i] = kc;
                        zc[i] = sz[par][c];
                        yc[i] = sy[par][c];
                        kn += kc * kc;
                        uz += uc * zc[i];
                        zkr += zc[i] * kc;
                    }
                }
                const float rk = __builtin_amdgcn_rsqf(wave_sum(kn));
                const float rden = 1.f / (1.f + wave_sum(uz));
                const float zk = wave_sum(zkr) * rk * rden;   // (z . k^) / (1 + u.z)
                // A_t k^ = A_{t-1} k^ - z (z . k^) / (1 + u.z)
                float ny = 0.f;
#pragma unroll
                for (int i = 0; i < NC64; ++i) {
                    yc[i] = yc[i] * rk - zc[i] * zk;
                    ny += yc[i] * yc[i];
                }
                const float ra = __builtin_amdgcn_rsqf(wave_sum(ny));
                if (wave == 0) {
#pragma unroll
                    for (int i = 0; i < NC64; ++i) {
                        const int c = lane + 64 * i;
                        if (DK % 64 == 0 || c < DK) sa[par][c] = yc[i] * ra;
                    }
                    if (lane == 0) srk[par] = rk;
                    if (ratio) {
                        // n_t = n_{t-1} + (1 - n_{t-1}.k^) a_t, then n_t . phi(q_t) for the readout
                        float nk = 0.f;
#pragma unroll
                        for (int i = 0; i < NC64; ++i) nk += nv[i] * kcol[i];
                        const float f = 1.f - wave_sum(nk) * rk;
                        float nq = 0.f;
#pragma unroll
                        for (int i = 0; i < NC64; ++i) {
                            const int c = lane + 64 * i;
                            if (DK % 64 == 0 || c < DK) {
                                nv[i] += f * (yc[i] * ra);
                                nq += nv[i] * blk[j * DK + c];
                            }
                        }
                        nq = wave_sum(nq);
                        if (lane == 0) sden[par] = nq;
                    }
                }
                // rank-1 update of this lane's row slice
                const float f = zm * rden;
                const float* zv = &sz[par][c0];
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const f32x4 zz = *reinterpret_cast<const f32x4*>(zv + 4 * i);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[4 * i + e] -= f * zz[e];
                }
            }
        } else if (t > 0) {
            // the memory, one token behind: token t - 1 with a_{t-1}
            const int ts = t - 1;
            const float* blk = sblk[(ts / TB) & 1];
            const int j = ts & (TB - 1);
            const float* kr = blk + OK + j * DK + c0;
            const float* qr = blk + j * DK + c0;
            const float vm = blk[OV + j * DV + m];
            float ep = 0.f;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const f32x4 kk = *reinterpret_cast<const f32x4*>(kr + 4 * i);
#pragma unroll
                for (int e = 0; e < 4; ++e) ep += x[4 * i + e] * kk[e];
            }
            const float d = vm - cross_row_sum(ep) * srk[ts & 1];   // v_m - (S k^)_m
            const float* av = &sa[ts & 1][c0];
            float op = 0.f;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const f32x4 aa = *reinterpret_cast<const f32x4*>(av + 4 * i);
                const f32x4 qq = *reinterpret_cast<const f32x4*>(qr + 4 * i);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[4 * i + e] += d * aa[e];
                    op += x[4 * i + e] * qq[e];
                }
            }
            op = cross_row_sum(op);
            if (ratio) op = op / sden[ts & 1];
            if (g == 0) Store<TS>::store(og, static_cast<int64_t>(ts) * DV + m, op);
        }
    }

    // (the penalty, the same in every part, is written by part 0)
    float* dst = is_a ? (a_out && part == 0 ? a_out + (bh * DK + m) * DK + c0 : nullptr)
                      : (s_out ? s_out + (bh * DV + m) * DK + c0 : nullptr);
    if (dst) {
#pragma unroll
        for (int i = 0; i < NQ; ++i)
            *reinterpret_cast<f32x4*>(dst + 4 * i) = f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]};
    }
    if (ratio && wave == 0 && part == 0 && n_out != nullptr) {
#pragma unroll
        for (int i = 0; i < NC64; ++i) {
            const int c = lane + 64 * i;
            if (DK % 64 == 0 || c < DK) n_out[bh * DK + c] = nv[i];
        }
    }
}

template <typename TS, int DK, int DV, int SPL>
hipError_t launch_split(const VlaArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    hipLaunchKernelGGL((vla_kernel<TS, DK, DV, SPL>), dim3(static_cast<unsigned>(heads * SPL)),
                       dim3(VlaShape<TS, DK, DV, SPL>::NT), 0, stream, static_cast<const TS*>(a.q),
                       static_cast<const TS*>(a.k), static_cast<const TS*>(a.v), static_cast<const TS*>(a.u),
                       a.inv_lambda0, a.a0, a.s0, a.n0, static_cast<TS*>(a.o), a.s_out, a.a_out, a.n_out,
                       a.ratio, a.T);
    return hipGetLastError();
}

// Two workgroups per sequence, each with half of the rows of S and the whole penalty chain,
// when there are fewer sequences than CUs: every CU then works, each on three quarters of a
// token's arithmetic. Not when the penalty is updated in place (a0 == a_out: a part could
// read it after another has written it; likewise the denominator vector) or d_v = 16.
template <typename TS, int DK, int DV>
hipError_t launch_shape(const VlaArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if constexpr (DV >= 32) {
        if (heads < 256 && (a.a_out == nullptr || a.a_out != a.a0) && (a.n_out == nullptr || a.n_out != a.n0))
            return launch_split<TS, DK, DV, 2>(a, stream);
    }
    return launch_split<TS, DK, DV, 1>(a, stream);
}

template <typename TS, int DK>
hipError_t launch_dk(const VlaArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_shape<TS, DK, 16>(a, stream);
        case 32: return launch_shape<TS, DK, 32>(a, stream);
        case 64: return launch_shape<TS, DK, 64>(a, stream);
        case 128: return launch_shape<TS, DK, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <typename TS>
hipError_t launch_typed(const VlaArgs& a, hipStream_t stream) {
    if (static_cast<int64_t>(a.B) * a.H == 0) return hipSuccess;
    switch (a.dk) {
        case 16: return launch_dk<TS, 16>(a, stream);
        case 32: return launch_dk<TS, 32>(a, stream);
        case 64: return launch_dk<TS, 64>(a, stream);
        case 128: return launch_dk<TS, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_vla(bool bf16, const VlaArgs& a, hipStream_t stream) {
    return bf16 ? launch_typed<unsigned short>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace glr
