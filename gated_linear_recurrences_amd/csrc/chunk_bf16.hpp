// Chunkwise forward with bfloat16 storage: bf16 MFMA (v_mfma_f32_16x16x32_bf16)
// for every contraction, fp32 accumulation, fp32 memory carried in registers.
//
// Method. The chunkwise form of "Le architetture lineari: RetNet, RWKV,
// xLSTM" (section "RetNet: la retention e le sue tre forme", Fig. 16.5): the
// masked-decay triangle inside a chunk of C tokens, the memory S carried from
// chunk to chunk. With local index i, j in [0, n), incoming memory S_in and local
// inclusive cumulative log-gates:
//
//   retention  P_ij = g^(i-j) (q_i.k_j)  (j <= i)
//              o_i = sum_j P_ij v_j + g^(i+1) S_in q_i
//              S_out = g^n S_in + sum_j g^(n-1-j) v_j k_j^T
//   GLA        P_ij = sum_c q_ic k_jc e^(b_ic - b_jc)
//              o_i = sum_j P_ij v_j + S_in (q_i . e^(b_i))
//              S_out = S_in Diag(e^(b_{n-1})) + sum_j v_j (k_j . e^(b_{n-1} - b_j))^T
//   gated delta ("Scrivere meglio nella memoria", sections "Correggere: la
//              delta rule" and "Unire oblio e correzione"; WY form):
//              A = strictly_lower(diag(beta) (K K^T . Gamma)), Gamma_ij = e^(G_i - G_j)
//              T = (I + A)^-1,  W = T diag(beta e^G) K,  U0 = T diag(beta) V
//              U = U0 - W S_in^T
//              o_i = e^(G_i) S_in q_i + sum_{j<=i} Gamma_ij (q_i.k_j) u_j
//              S_out = e^(G_{n-1}) S_in + sum_j e^(G_{n-1} - G_j) u_j k_j^T
//
// Work decomposition (gfx950). The gates multiply S from the right, so each row
// of S (a value channel) evolves on its own: a workgroup owns one (batch, head)
// and DVT = 16 * NW value channels, and wave w owns 16 of them for the whole
// sequence - its slice of S^T (d_k x 16, fp32) lives in that wave's MFMA
// accumulators and never leaves registers between chunks. Per chunk:
//   staging   q, k, v (and gates) of chunk c+1 are fetched from HBM into
//             registers while chunk c computes (16-byte coalesced loads), then
//             written to LDS in the layouts the MFMA operands need (token-major
//             q, k; channel-major k^T and v^T, decay weights folded in);
//   phase 1   the S-independent triangle: P (and the delta rule's A) tiles on
//             MFMA, spread over the waves, written to LDS;
//   (delta)   T's 16x16 diagonal blocks by forward substitution (one wave),
//             then W and U0 by blocked forward substitution on MFMA;
//   chain     per wave, the only S-dependent work: S q readout, P V (or P U),
//             and the state update K^T V, all on MFMA against the register-
//             resident S.
// The MFMA k-slot assignment used throughout is the "split" one: within a
// 32-wide reduction block, lane (r, g) feeds indices 4g..4g+3 of the block's
// first 16 and 4g..4g+3 of its second 16 - exactly what a 16x16 accumulator
// tile holds per lane, so S^T and U feed the next MFMA straight from registers.
// Cumulative log-gates are kept in log2 units and exponentiated with v_exp_f32.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace glr {
namespace bf16k {

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

__device__ __forceinline__ bf16x4 cvt4(f32x4 x) {
    bf16x4 r;
    r[0] = static_cast<__bf16>(x[0]); r[1] = static_cast<__bf16>(x[1]);
    r[2] = static_cast<__bf16>(x[2]); r[3] = static_cast<__bf16>(x[3]);
    return r;
}

__device__ __forceinline__ f32x4 zf4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

__device__ __forceinline__ f32x4 mfma16k(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Operand from a row-major LDS array X (row stride RS elements) for reduction block kb:
// split k-slots, the second half zero when the reduction has only 2*kb+1 tiles.
template <int NTILE, int RS>
__device__ __forceinline__ bf16x8 split_op(const u16* X, int row, int kb, int g) {
    const u16* p = X + row * RS + 32 * kb + 4 * g;
    return join8(ld4(p), (2 * kb + 1 < NTILE) ? ld4(p + 16) : zero4());
}

__device__ __forceinline__ u16 bits(__bf16 x) { return __builtin_bit_cast(u16, x); }

template <int VARIANT, int C, int DK, int NW>
__global__ __launch_bounds__(64 * NW)
void chunk_kernel(Params p) {
    constexpr int NT = 64 * NW;
    constexpr int DVT = 16 * NW;
    constexpr int CT = C / 16;           // 16-token tiles per chunk
    constexpr int KT = DK / 16;          // 16-channel tiles of the key dimension
    constexpr int KB = (KT + 1) / 2;     // 32-wide reduction blocks over d_k
    constexpr int JB = (CT + 1) / 2;     // 32-wide reduction blocks over the chunk
    constexpr int QS = DK + 8;           // row stride of token-major bf16 arrays
    constexpr int TS = C + 8;            // row stride of channel-major bf16 arrays
    constexpr int AS = C + 4;            // row stride of the fp32 triangular system
    constexpr int BS = DK + 4;           // row stride of the fp32 cumulative gates
    constexpr bool kGla = VARIANT == kGLA;
    constexpr bool kDel = VARIANT == kGDelta;

    __shared__ __align__(16) u16 sQ[C * QS];
    __shared__ __align__(16) u16 sK[C * QS];
    __shared__ __align__(16) u16 sKT[DK * TS];
    __shared__ __align__(16) u16 sVT[DVT * TS];
    __shared__ __align__(16) u16 sP[C * TS];
    __shared__ __align__(16) u16 sQe[kGla ? C * QS : 8];
    __shared__ __align__(16) float sB[kGla ? C * BS : 4];
    // GLA factor tables: F[it][jt][c], Z[t][c], L[t][c], decay[c]
    __shared__ __align__(16) float sTab[kGla ? (CT * CT + 2 * CT + 1) * DK : 4];
    __shared__ __align__(16) float sA[kDel ? C * AS : 4];
    __shared__ __align__(16) float sD[kDel ? CT * 256 : 4];
    __shared__ __align__(16) u16 sW[kDel ? C * QS : 8];
    __shared__ __align__(16) float sG[C];
    __shared__ __align__(16) float sBeta[C];
    float* const tabF = sTab;
    float* const tabZ = sTab + CT * CT * DK;
    float* const tabL = tabZ + CT * DK;
    float* const tabDec = tabL + CT * DK;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int g = lane >> 4;

    // XCD-aware order: consecutive workgroup ids land on different XCDs, so the
    // value-channel tiles of one head are given ids that share an XCD (and its L2).
    int L = blockIdx.x;
    if (p.remap) L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int bh = L / p.tiles;
    const int v0 = (L % p.tiles) * DVT;
    const int h = bh % p.H;
    const int T = p.T;
    const int dv = p.dv;
    const int64_t tok0 = static_cast<int64_t>(bh) * T;
    const u16* qg = p.q + tok0 * DK;
    const u16* kg = p.k + tok0 * DK;
    const u16* vg = p.v + tok0 * dv + v0;
    u16* og = p.o + tok0 * dv + v0;
    const float lg2 = (VARIANT == kRetention) ? p.gate[h] * kLog2e : 0.f;

    // ---- the wave's slice of the memory, S^T[c][m]: sacc[ct][r] = S[v0+16w+r16][16ct+4g+r]
    f32x4 sacc[KT];
    {
        const float* srow = p.s0 ? p.s0 + (static_cast<int64_t>(bh) * dv + v0 + 16 * w + r16) * DK : nullptr;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
            sacc[ct] = srow ? *reinterpret_cast<const f32x4*>(srow + 16 * ct + 4 * g) : zf4();
    }

    // ---- register staging of one chunk (4-row x 8-column micro-tiles, 16-byte loads)
    constexpr int QK_ITEMS = (C / 4) * (DK / 8);
    constexpr int QK_PER = (QK_ITEMS + NT - 1) / NT;
    constexpr int V_ITEMS = (C / 4) * (DVT / 8);
    constexpr int V_PER = (V_ITEMS + NT - 1) / NT;
    constexpr int G_ITEMS = kGla ? (C / 4) * (DK / 4) : 0;
    constexpr int G_PER = kGla ? (G_ITEMS + NT - 1) / NT : 1;
    u16x8 rq[QK_PER][4], rk[QK_PER][4], rv[V_PER][4];
    f32x4 rg[G_PER][4];
    float rla = 0.f, rbe = 0.f;

    auto fetch = [&](int t0, int n) {
#pragma unroll
        for (int pi = 0; pi < QK_PER; ++pi) {
            const int item = tid + pi * NT;
            if (item < QK_ITEMS) {
                const int row0 = (item / (DK / 8)) * 4, col0 = (item % (DK / 8)) * 8;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const bool in = row0 + rr < n;
                    const int64_t off = static_cast<int64_t>(t0 + row0 + rr) * DK + col0;
                    u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
                    rq[pi][rr] = in ? *reinterpret_cast<const u16x8*>(qg + off) : z;
                    rk[pi][rr] = in ? *reinterpret_cast<const u16x8*>(kg + off) : z;
                }
            }
        }
#pragma unroll
        for (int pi = 0; pi < V_PER; ++pi) {
            const int item = tid + pi * NT;
            if (item < V_ITEMS) {
                const int row0 = (item / (DVT / 8)) * 4, col0 = (item % (DVT / 8)) * 8;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
                    rv[pi][rr] = (row0 + rr < n)
                        ? *reinterpret_cast<const u16x8*>(vg + static_cast<int64_t>(t0 + row0 + rr) * dv + col0)
                        : z;
                }
            }
        }
        if constexpr (kGla) {
            const float* gg = p.gate + tok0 * DK;
#pragma unroll
            for (int pi = 0; pi < G_PER; ++pi) {
                const int item = tid + pi * NT;
                if (item < G_ITEMS) {
                    const int row0 = (item / (DK / 4)) * 4, col0 = (item % (DK / 4)) * 4;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        rg[pi][rr] = (row0 + rr < n)
                            ? *reinterpret_cast<const f32x4*>(gg + static_cast<int64_t>(t0 + row0 + rr) * DK + col0)
                            : zf4();
                }
            }
        }
        if constexpr (kDel) {
            if (tid < C) {
                const bool in = tid < n;
                rla = in ? p.gate[tok0 + t0 + tid] : 0.f;
                rbe = in ? p.beta[tok0 + t0 + tid] : 0.f;
            }
        }
    };

    // v^T (raw) into LDS: shared by all variants
    auto stage_v = [&]() {
#pragma unroll
        for (int pi = 0; pi < V_PER; ++pi) {
            const int item = tid + pi * NT;
            if (item < V_ITEMS) {
                const int row0 = (item / (DVT / 8)) * 4, col0 = (item % (DVT / 8)) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    u16x4 t = {rv[pi][0][e], rv[pi][1][e], rv[pi][2][e], rv[pi][3][e]};
                    *reinterpret_cast<u16x4*>(sVT + (col0 + e) * TS + row0) = t;
                }
            }
        }
    };

    const int n_chunks = (T + C - 1) / C;
    if (n_chunks > 0) fetch(0, T < C ? T : C);

    for (int ch = 0; ch < n_chunks; ++ch) {
        const int t0 = ch * C;
        const int n = (T - t0 < C) ? (T - t0) : C;
        __syncthreads();  // every wave is done with the previous chunk's LDS

        // ------------------------------------------------------------ staging
        stage_v();
        if constexpr (!kGla) {
#pragma unroll
            for (int pi = 0; pi < QK_PER; ++pi) {
                const int item = tid + pi * NT;
                if (item < QK_ITEMS) {
                    const int row0 = (item / (DK / 8)) * 4, col0 = (item % (DK / 8)) * 8;
                    float wgt[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        *reinterpret_cast<u16x8*>(sQ + (row0 + rr) * QS + col0) = rq[pi][rr];
                        *reinterpret_cast<u16x8*>(sK + (row0 + rr) * QS + col0) = rk[pi][rr];
                        const int j = row0 + rr;
                        // retention folds the carry weight g^(n-1-j) into k^T; the delta rule
                        // applies its weights to U in registers
                        wgt[rr] = (VARIANT == kRetention) ? ((j < n) ? ex2(static_cast<float>(n - 1 - j) * lg2) : 0.f)
                                                          : 1.f;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        bf16x4 t;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            t[rr] = static_cast<__bf16>(bf16_bits_to_f32(rk[pi][rr][e]) * wgt[rr]);
                        st4(sKT + (col0 + e) * TS + row0, t);
                    }
                }
            }
            if constexpr (kDel) {
                if (w == 0) {
                    float x = (lane < C) ? rla * kLog2e : 0.f;
                    x = wave_inclusive_scan(x);
                    if (lane < C) { sG[lane] = x; sBeta[lane] = rbe; }
                }
            }
        } else {
            // GLA: raw log-gates (log2 units) -> sB, then per-channel wavefront scans
#pragma unroll
            for (int pi = 0; pi < G_PER; ++pi) {
                const int item = tid + pi * NT;
                if (item < G_ITEMS) {
                    const int row0 = (item / (DK / 4)) * 4, col0 = (item % (DK / 4)) * 4;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        *reinterpret_cast<f32x4*>(sB + (row0 + rr) * BS + col0) = rg[pi][rr] * kLog2e;
                }
            }
            __syncthreads();
            for (int c = w; c < DK; c += NW) {
                float x = (lane < C) ? sB[lane * BS + c] : 0.f;
                x = wave_inclusive_scan(x);
                if (lane < C) sB[lane * BS + c] = x;
            }
            __syncthreads();
            // factor tables per key channel; reference point of token tile t is the
            // cumulative gate just before it (0 for the first tile)
            for (int c = tid; c < DK; c += NT) {
                float ref[CT];
#pragma unroll
                for (int t = 0; t < CT; ++t) ref[t] = (t == 0) ? 0.f : sB[(16 * t - 1) * BS + c];
                const float last = sB[(C - 1) * BS + c];
#pragma unroll
                for (int it = 0; it < CT; ++it) {
#pragma unroll
                    for (int jt = 0; jt < it; ++jt) tabF[(it * CT + jt) * DK + c] = ex2(ref[it] - ref[jt]);
                    tabZ[it * DK + c] = ex2(ref[it]);
                    tabL[it * DK + c] = ex2(last - ref[it]);
                }
                tabDec[c] = ex2(last);
            }
            __syncthreads();
            // rescaled q, q e^b, k, and the carry-weighted k^T
#pragma unroll
            for (int pi = 0; pi < QK_PER; ++pi) {
                const int item = tid + pi * NT;
                if (item < QK_ITEMS) {
                    const int row0 = (item / (DK / 8)) * 4, col0 = (item % (DK / 8)) * 8;
                    const int t = row0 / 16;
                    float ref[8], zf[8], lf[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ref[e] = (t == 0) ? 0.f : sB[(16 * t - 1) * BS + col0 + e];
                        zf[e] = tabZ[t * DK + col0 + e];
                        lf[e] = tabL[t * DK + col0 + e];
                    }
                    float kd[4][8];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int i = row0 + rr;
                        u16x8 oq, oqe, ok;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float b = sB[i * BS + col0 + e];
                            const float E = ex2(b - ref[e]);
                            const float Ei = ex2(ref[e] - b);
                            const float qx = bf16_bits_to_f32(rq[pi][rr][e]) * E;
                            kd[rr][e] = bf16_bits_to_f32(rk[pi][rr][e]) * Ei;
                            oq[e] = bits(static_cast<__bf16>(qx));
                            oqe[e] = bits(static_cast<__bf16>(qx * zf[e]));
                            ok[e] = bits(static_cast<__bf16>(kd[rr][e]));
                        }
                        *reinterpret_cast<u16x8*>(sQ + i * QS + col0) = oq;
                        *reinterpret_cast<u16x8*>(sQe + i * QS + col0) = oqe;
                        *reinterpret_cast<u16x8*>(sK + i * QS + col0) = ok;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        bf16x4 tt;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) tt[rr] = static_cast<__bf16>(kd[rr][e] * lf[e]);
                        st4(sKT + (col0 + e) * TS + row0, tt);
                    }
                }
            }
        }
        __syncthreads();

        // chunk ch is in LDS: fetch the next one while this one computes
        if (ch + 1 < n_chunks) {
            const int t1 = t0 + C;
            fetch(t1, (T - t1 < C) ? (T - t1) : C);
        }

        // ------------------------------------------------------------ phase 1: the triangle
        constexpr int NPAIR = CT * (CT + 1) / 2;
        for (int pr = w; pr < NPAIR; pr += NW) {
            int it = 0, jt = pr;
            while (jt > it) { jt -= it + 1; ++it; }
            f32x4 acc = zf4(), acc2 = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 a = split_op<KT, QS>(sK, 16 * jt + r16, kb, g);
                bf16x8 bq = split_op<KT, QS>(sQ, 16 * it + r16, kb, g);
                if constexpr (kGla) {
                    if (jt < it) {
                        const float* F = tabF + (it * CT + jt) * DK + 32 * kb + 4 * g;
                        const f32x4 flo = *reinterpret_cast<const f32x4*>(F);
                        const f32x4 fhi = (2 * kb + 1 < KT) ? *reinterpret_cast<const f32x4*>(F + 16) : zf4();
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            bq[e] = static_cast<__bf16>(static_cast<float>(bq[e]) * flo[e]);
                            bq[4 + e] = static_cast<__bf16>(static_cast<float>(bq[4 + e]) * fhi[e]);
                        }
                    }
                }
                acc = mfma_16x16x32(a, bq, acc);
                if constexpr (kDel) acc2 = mfma_16x16x32(a, split_op<KT, QS>(sK, 16 * it + r16, kb, g), acc2);
            }
            // acc[r] = sum_c k[j][c] q[i][c] with j = 16jt + 4g + r, i = 16it + r16
            const int i = 16 * it + r16;
            bf16x4 pv;
            f32x4 av;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jt + 4 * g + r;
                float val = 0.f, aval = 0.f;
                if (j <= i) {
                    if constexpr (VARIANT == kRetention) {
                        val = acc[r] * ex2(static_cast<float>(i - j) * lg2);
                    } else if constexpr (kGla) {
                        val = acc[r];
                    } else {
                        const float gam = ex2(sG[i] - sG[j]);
                        val = acc[r] * gam;
                        aval = (j < i) ? sBeta[i] * acc2[r] * gam : 0.f;
                    }
                }
                pv[r] = static_cast<__bf16>(val);
                av[r] = aval;
            }
            st4(sP + i * TS + 16 * jt + 4 * g, pv);
            if constexpr (kDel) *reinterpret_cast<f32x4*>(sA + i * AS + 16 * jt + 4 * g) = av;
        }
        __syncthreads();

        // the wave's memory slice as bf16 MFMA operands (split k-slots over d_k)
        bf16x8 sop[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            sop[kb] = join8(cvt4(sacc[2 * kb]), (2 * kb + 1 < KT) ? cvt4(sacc[2 * kb + 1]) : zero4());

        // readout of the incoming memory, q_i S^T (rows i = 16it + 4g + r, column m = r16)
        const u16* qsrc = kGla ? sQe : sQ;
        f32x4 oe[CT];
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            f32x4 acc = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc = mfma_16x16x32(split_op<KT, QS>(qsrc, 16 * it + r16, kb, g), sop[kb], acc);
            oe[it] = acc;
        }

        f32x4 U[kDel ? CT : 1];
        if constexpr (kDel) {
            // ---------------------------------------------------- T's diagonal 16x16 blocks
            if (w == 0) {
                const int b = lane >> 4, j = lane & 15;
                if (b < CT) {
                    float x[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float* arow = sA + (16 * b + i) * AS + 16 * b;
                        float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
                        for (int kk = 0; kk < i; ++kk) acc -= arow[kk] * x[kk];
                        x[i] = acc;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) sD[b * 256 + i * 16 + j] = x[i];
                }
            }
            __syncthreads();
            // ---------------------------------------------------- blocked forward substitution
            // X_b = D_b (R_b - sum_{kk<b} A_{b,kk} X_kk) for the right-hand sides
            // diag(beta e^G) K (-> W, LDS) and diag(beta) V (-> U0, registers)
            auto solve = [&](auto rhs, f32x4 (&X)[CT]) {
#pragma unroll
                for (int b = 0; b < CT; ++b) {
                    f32x4 acc = rhs(b);
#pragma unroll
                    for (int kk = 0; kk < b; ++kk) {
                        const f32x4 a = *reinterpret_cast<const f32x4*>(sA + (16 * b + r16) * AS + 16 * kk + 4 * g);
                        acc = mfma16k(cvt4(-a), cvt4(X[kk]), acc);
                    }
                    const f32x4 d = *reinterpret_cast<const f32x4*>(sD + b * 256 + r16 * 16 + 4 * g);
                    X[b] = mfma16k(cvt4(d), cvt4(acc), zf4());
                }
            };
            for (int nt = w; nt < KT; nt += NW) {
                f32x4 X[CT];
                solve([&](int b) {
                    const bf16x4 kv = ld4(sKT + (16 * nt + r16) * TS + 16 * b + 4 * g);
                    f32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = 16 * b + 4 * g + e;
                        r[e] = static_cast<float>(kv[e]) * sBeta[j] * ex2(sG[j]);
                    }
                    return r;
                }, X);
#pragma unroll
                for (int b = 0; b < CT; ++b)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sW[(16 * b + 4 * g + e) * QS + 16 * nt + r16] = bits(static_cast<__bf16>(X[b][e]));
            }
            solve([&](int b) {
                const bf16x4 vv = ld4(sVT + (16 * w + r16) * TS + 16 * b + 4 * g);
                f32x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(vv[e]) * sBeta[16 * b + 4 * g + e];
                return r;
            }, U);
            __syncthreads();
            // ---------------------------------------------------- U = U0 - W S^T (on the chain)
#pragma unroll
            for (int b = 0; b < CT; ++b) {
                f32x4 acc = zf4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) acc = mfma_16x16x32(split_op<KT, QS>(sW, 16 * b + r16, kb, g), sop[kb], acc);
                U[b] = U[b] - acc;
            }
        }

        // ------------------------------------------------------------ outputs
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            f32x4 oi = zf4();
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if (2 * jb <= it) {
                    const bool hi = 2 * jb + 1 <= it;
                    const u16* prow = sP + (16 * it + r16) * TS + 32 * jb + 4 * g;
                    const bf16x8 a = join8(ld4(prow), hi ? ld4(prow + 16) : zero4());
                    bf16x8 b;
                    if constexpr (kDel) {
                        b = join8(cvt4(U[2 * jb]), hi ? cvt4(U[2 * jb + 1]) : zero4());
                    } else {
                        const u16* vrow = sVT + (16 * w + r16) * TS + 32 * jb + 4 * g;
                        b = join8(ld4(vrow), hi ? ld4(vrow + 16) : zero4());
                    }
                    oi = mfma_16x16x32(a, b, oi);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + 4 * g + r;
                float scale = 1.f;
                if constexpr (VARIANT == kRetention) scale = ex2(static_cast<float>(i + 1) * lg2);
                if constexpr (kDel) scale = ex2(sG[i]);
                if (i < n)
                    og[static_cast<int64_t>(t0 + i) * dv + 16 * w + r16] =
                        bits(static_cast<__bf16>(oi[r] + scale * oe[it][r]));
            }
        }

        // ------------------------------------------------------------ memory carried on
        if constexpr (kDel) {
            const float glast = sG[C - 1];   // padded tail tokens have log-gate 0
            const float dec = ex2(glast);
            f32x4 wU[CT];
#pragma unroll
            for (int b = 0; b < CT; ++b)
#pragma unroll
                for (int e = 0; e < 4; ++e) wU[b][e] = U[b][e] * ex2(glast - sG[16 * b + 4 * g + e]);
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                f32x4 acc = sacc[ct] * dec;
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    const bool hi = 2 * jb + 1 < CT;
                    const u16* krow = sKT + (16 * ct + r16) * TS + 32 * jb + 4 * g;
                    acc = mfma_16x16x32(join8(ld4(krow), hi ? ld4(krow + 16) : zero4()),
                                        join8(cvt4(wU[2 * jb]), hi ? cvt4(wU[2 * jb + 1]) : zero4()), acc);
                }
                sacc[ct] = acc;
            }
        } else {
            const float dec_all = (VARIANT == kRetention) ? ex2(static_cast<float>(n) * lg2) : 1.f;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                f32x4 acc;
                if constexpr (kGla) {
                    const f32x4 d = *reinterpret_cast<const f32x4*>(tabDec + 16 * ct + 4 * g);
                    acc = sacc[ct] * d;
                } else {
                    acc = sacc[ct] * dec_all;
                }
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    const bool hi = 2 * jb + 1 < CT;
                    const u16* krow = sKT + (16 * ct + r16) * TS + 32 * jb + 4 * g;
                    const u16* vrow = sVT + (16 * w + r16) * TS + 32 * jb + 4 * g;
                    acc = mfma_16x16x32(join8(ld4(krow), hi ? ld4(krow + 16) : zero4()),
                                        join8(ld4(vrow), hi ? ld4(vrow + 16) : zero4()), acc);
                }
                sacc[ct] = acc;
            }
        }
    }

    if (p.s_out) {
        float* srow = p.s_out + (static_cast<int64_t>(bh) * dv + v0 + 16 * w + r16) * DK;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) *reinterpret_cast<f32x4*>(srow + 16 * ct + 4 * g) = sacc[ct];
    }
}

template <int VARIANT, int C, int DK, int NW>
hipError_t launch_nw(const ChunkArgs& a, hipStream_t stream) {
    constexpr int DVT = 16 * NW;
    Params p;
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.gate = a.gate;
    p.beta = a.beta;
    p.s0 = a.s0;
    p.o = static_cast<u16*>(a.o);
    p.s_out = a.s_out;
    p.H = a.H;
    p.T = a.T;
    p.dv = a.dv;
    p.tiles = a.dv / DVT;
    const int64_t G = static_cast<int64_t>(a.B) * a.H * p.tiles;
    p.remap = (G % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_kernel<VARIANT, C, DK, NW>), dim3(static_cast<unsigned>(G)), dim3(64 * NW), 0,
                       stream, p);
    return hipGetLastError();
}

template <int VARIANT, int C, int DK>
hipError_t launch_dk(const ChunkArgs& a, hipStream_t stream) {
    if (a.dv >= 64) return launch_nw<VARIANT, C, DK, 4>(a, stream);
    if (a.dv == 32) return launch_nw<VARIANT, C, DK, 2>(a, stream);
    return launch_nw<VARIANT, C, DK, 1>(a, stream);
}

template <int VARIANT, int C>
hipError_t launch_c(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_dk<VARIANT, C, 16>(a, stream);
        case 32: return launch_dk<VARIANT, C, 32>(a, stream);
        case 64: return launch_dk<VARIANT, C, 64>(a, stream);
        case 128: return launch_dk<VARIANT, C, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int VARIANT>
hipError_t launch_variant(const ChunkArgs& a, hipStream_t stream) {
    switch (a.chunk) {
        case 16: return launch_c<VARIANT, 16>(a, stream);
        case 32: return launch_c<VARIANT, 32>(a, stream);
        case 64: return launch_c<VARIANT, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace bf16k
}  // namespace glr
