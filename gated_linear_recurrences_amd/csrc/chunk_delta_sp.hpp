// Gated delta rule, chunk 64, bf16 storage: a chunk-parallel prep and a single pass that
// keeps the memory on chip.
//
// Method: the gated delta rule ("Scrivere meglio nella memoria", section "Unire oblio e
// correzione: Gated DeltaNet") in the chunkwise form of the RetNet page (section "RetNet:
// la retention e le sue tre forme", Fig. 16.5), with the pseudo-values of the UT
// representation (section "Correggere: la delta rule": one triangular system per chunk,
// only the end-of-chunk memory passed on). Per chunk of n tokens with local inclusive
// cumulative log-gates G and Gamma_ij = e^(G_i - G_j):
//   A     = strictly_lower(diag(beta) (K K^T . Gamma)),   T_U = (I + A)^-1 diag(beta)
//   U     = T_U (V - diag(e^G) K S_in^T)
//   o_i   = e^(G_i) S_in q_i + sum_{j<=i} Gamma_ij (q_i.k_j) u_j
//   S_out = e^(G_{n-1}) S_in + sum_j e^(G_{n-1} - G_j) u_j k_j^T
// T_U depends only on the chunk's keys, gates and write strengths, so:
//   prep         (all chunks in parallel) G and T_U (bf16, lower triangular) to the
//                workspace: 8.25 KB per (sequence, chunk); with DeltaNet's feature map fused
//                in, also q and k mapped by SiLU then L2 normalisation per token;
//   single pass  (chunks in order) one workgroup per (sequence, 16 NV value channels);
//   row norm     (with DeltaNet's output norm fused in) every output row RMS-normalised in
//                place, one wave per four rows.
//
// Single pass, four waves. Rows of S (value channels) evolve independently, so wave vt < NV
// (a "chain" wave) owns 16 value channels and keeps S^T for them (every key) in fp32 MFMA
// accumulators; each product of the chain takes the previous one's accumulators directly as
// its B operand (bf16, a fixed permutation of the reduction slots), with nothing exchanged
// between waves:
//   Y = K S_in^T           (reduction over keys; K rows from LDS)
//   R = V - diag(e^G) Y,   U = T_U R    (reduction over tokens; T_U rows from LDS)
//   S^T <- e^(G_last) S^T + K^T diag(e^(G_last - G)) U    (K^T by ds_read_b64_tr_b16)
// and hands S_in (bf16 rows) and U (a bf16 hi + lo pair) over in LDS. Waves 2 and 3 (the
// "output" waves) finish the previous chunk from that hand-off: each takes two token tiles
// ({0, 3} and {1, 2}: five triangle tiles each) for every value tile of the workgroup,
//   P = (Q K^T . Gamma) masked,   o^T = S_in Q^T diag(e^G) + U^T P^T,
// with its q rows loaded from HBM straight into registers (MFMA operand layout) a chunk
// ahead. Operands (K, the v slice, T_U, G) are loaded two chunks ahead into a register ring
// by every lane and written to LDS just before the chunk's barrier; K and the gate tables
// live in three LDS slots (staged, the chain's chunk, the output's chunk), the rest in two.
// One workgroup barrier per chunk. The value slices of one sequence get block ids on one XCD
// and share its L2 copy of K, q and T_U.
#pragma once

#include <type_traits>

#include "chunk_delta.hpp"

namespace glr {
namespace ck {

// Workspace: per (sequence, chunk) T_U [C][C] bf16 (row = token i, lower triangular with the
// write strengths folded into its columns, zero above the diagonal) and G [C] fp32 (log2
// units; flat past the end of a short last chunk), each array contiguous over the chunks;
// with the feature map fused in, then the mapped keys and queries [C][DK] bf16 per chunk.
inline size_t dsp_ws_bytes(int64_t chunks, int C, int dk, bool mapped) {
    return delta_ws_align(chunks * C * C * 2) + delta_ws_align(chunks * C * 4) +
           (mapped ? 2 * delta_ws_align(chunks * C * dk * 2) : 0);
}

struct DspParams {
    const u16* q;         // [BH][T][DK]
    const u16* k;         // [BH][T][DK]
    const u16* v;         // [BH][T][DV]
    const float* alpha;   // log alpha [BH][T]
    const float* beta;    // [BH][T]
    const float* s0;      // [BH][DV][DK] or null
    u16* o;               // [BH][T][DV]
    float* s_out;         // [BH][DV][DK] or null
    u16* tu;              // [BH * NC][C][C]
    float* g;             // [BH * NC][C]
    // feature map fused in: the raw projections (q and k above then point at the mapped
    // copies the prep writes, [BH * NC][C][DK] each)
    const u16* qraw;
    const u16* kraw;
    u16* qmap;
    u16* kmap;
    int T, NC, slices, remap, map;
    int qk_seq;           // tokens per sequence in q and k as read by the single pass: T, or
                          // NC * C for the mapped copies
};

// ====================================================================== prep
//
// One workgroup (four waves) per (sequence, chunk): stage k (mapped by SiLU + L2 first when
// the feature map is fused in, and q mapped beside it, both written to the workspace);
// cumulative log2-gates by a wavefront prefix scan; A tiles on MFMA (fp32); T's 16 x 16
// diagonal blocks by forward substitution (one wave); T's column blocks, one per wave
// (T_iw = -D_i sum_{w<=m<i} A_im T_mw); T_U = T diag(beta) through LDS to the workspace
// with 16-byte stores.
template <int C, int DK>
struct TfacLayout {
    static constexpr int CT = C / 16;
    static constexpr int KS = tile_stride(DK);
    static constexpr int AS = C + 4;
    static constexpr int TS = C + 8;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int oK = 0;
    static constexpr int oA = oK + al(C * KS * 2);
    static constexpr int oD = oA + al(C * AS * 4);
    static constexpr int oT = oD + al(CT * 256 * 4);
    static constexpr int oG = oT + al(C * TS * 2);
    static constexpr int oB = oG + al(C * 4);
    static constexpr int bytes = oB + al(C * 4);
    static_assert(bytes <= 64 * 1024, "LDS budget of the delta prep exceeded");
};

template <int C, int DK>
__global__ __launch_bounds__(256)
void delta_tfac_kernel(DspParams p) {
    using Lay = TfacLayout<C, DK>;
    constexpr int CT = C / 16, NT = 256, NW = 4;
    constexpr int KS = Lay::KS, AS = Lay::AS, TS = Lay::TS;
    constexpr int KB = (DK + 31) / 32;
    constexpr int KP = C * DK / 8, KP_PER = (KP + NT - 1) / NT;
    constexpr int TP = C * C / 8, TP_PER = (TP + NT - 1) / NT;
    constexpr int NPAIR = CT * (CT + 1) / 2;
    static_assert(CT <= NW, "one wave per column block of T");

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    float* const sA = reinterpret_cast<float*>(smem + Lay::oA);
    float* const sD = reinterpret_cast<float*>(smem + Lay::oD);
    u16* const sT = reinterpret_cast<u16*>(smem + Lay::oT);
    float* const sG = reinterpret_cast<float*>(smem + Lay::oG);
    float* const sBeta = reinterpret_cast<float*>(smem + Lay::oB);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
    const int T = p.T;
    const int t0 = c * C, n = (T - t0 < C) ? (T - t0) : C;
    const int64_t tok0 = static_cast<int64_t>(bh) * T + t0;
    const int64_t chunk = static_cast<int64_t>(bh) * p.NC + c;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};

    // ---- stage k (rows past the end zero); cumulative gates and write strengths
    static_assert(KP % NT == 0, "every lane holds whole pieces (the row map's shuffles need all lanes)");
    u16x8 rk[KP_PER];
    const u16* kin = p.map ? p.kraw : p.k;
#pragma unroll
    for (int i = 0; i < KP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        const unsigned off = (j < n) ? static_cast<unsigned>(j * DK + col) : 0u;
        rk[i] = *reinterpret_cast<const u16x8*>(kin + tok0 * DK + off);
    }
    if (p.map) {
        // DeltaNet's feature map on k and q: a row's DK / 8 pieces sit in one aligned lane group
        u16* const km = p.kmap + chunk * C * DK;
        u16* const qm = p.qmap + chunk * C * DK;
#pragma unroll
        for (int i = 0; i < KP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const unsigned off = (j < n) ? static_cast<unsigned>(j * DK + col) : 0u;
            const u16x8 qx = silu_l2_piece<DK / 8>(*reinterpret_cast<const u16x8*>(p.qraw + tok0 * DK + off));
            rk[i] = silu_l2_piece<DK / 8>(rk[i]);
            *reinterpret_cast<u16x8*>(km + j * DK + col) = (j < n) ? rk[i] : z8;
            *reinterpret_cast<u16x8*>(qm + j * DK + col) = (j < n) ? qx : z8;
        }
    }
    if (w == 0) {
        float la = 0.f, be = 0.f;
        if (lane < n) {
            la = p.alpha[tok0 + lane] * kLog2e;
            be = p.beta[tok0 + lane];
        }
        const float G = wave_inclusive_scan(la);   // padded tokens add a zero log-gate
        if (lane < C) {
            sG[lane] = G;
            sBeta[lane] = be;
            p.g[chunk * C + lane] = G;
        }
    }
#pragma unroll
    for (int i = 0; i < KP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        *reinterpret_cast<u16x8*>(sK + j * KS + col) = (j < n) ? rk[i] : z8;
    }
    lds_barrier();

    // ---- A = strictly_lower(diag(beta) (K K^T . Gamma)), tiles (it, jt <= it)
    for (int pr0 = w; pr0 < NPAIR; pr0 += NW) {
        int it = 0, jt = pr0;
        while (jt > it) { jt -= it + 1; ++it; }
        const int i = 16 * it + r16;
        f32x4 acc = zf4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            bf16x8 ka = as_bf16x8(z8), kb8 = as_bf16x8(z8);
            if (col < DK) {
                ka = *reinterpret_cast<const bf16x8*>(sK + (16 * jt + r16) * KS + col);
                kb8 = *reinterpret_cast<const bf16x8*>(sK + i * KS + col);
            }
            acc = mfma_16x16x32(ka, kb8, acc);
        }
        // acc[r] = k_i . k_j, j = 16jt + 4g + r
        const float gi = sG[i], bi = sBeta[i];
        const f32x4 gj = ldf4(sG + 16 * jt + 4 * g);
        f32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * g + r;
            a[r] = (j < i) ? bi * acc[r] * ex2(gi - gj[r]) : 0.f;
        }
        stf4(sA + i * AS + 16 * jt + 4 * g, a);
    }
    lds_barrier();

    // ---- T's diagonal 16 x 16 blocks D_b = (I + A_bb)^-1 by forward substitution: lane
    // (b, j) computes column j of block b
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
    lds_barrier();

    // ---- column block w of T: lane (r16, g) holds T[16i + 4g + r][16w + r16]; written as
    // T_U (times the column's write strength), zero above the diagonal blocks
    if (w < CT) {
        const float fu = sBeta[16 * w + r16];
        f32x4 tcol[CT];
#pragma unroll
        for (int i = 0; i < CT; ++i) {
            f32x4 t = zf4();
            if (i == w) {
#pragma unroll
                for (int r = 0; r < 4; ++r) t[r] = sD[w * 256 + (4 * g + r) * 16 + r16];
            } else if (i > w) {
                f32x4 acc = zf4();
#pragma unroll
                for (int m = 0; m < CT; ++m) {
                    if (m < w || m >= i) continue;
                    const f32x4 a = ldf4(sA + (16 * i + r16) * AS + 16 * m + 4 * g);
                    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cvt4(a), cvt4(tcol[m]), acc, 0, 0, 0);
                }
                const f32x4 d = ldf4(sD + i * 256 + r16 * 16 + 4 * g);
                t = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cvt4(-d), cvt4(acc), zf4(), 0, 0, 0);
            }
            tcol[i] = t;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sT[(16 * i + 4 * g + r) * TS + 16 * w + r16] = __builtin_bit_cast(u16, static_cast<__bf16>(t[r] * fu));
        }
    }
    lds_barrier();

    u16* const tg = p.tu + chunk * C * C;
#pragma unroll
    for (int i = 0; i < TP_PER; ++i) {
        const int idx = tid + i * NT;
        if (TP % NT == 0 || idx < TP) {
            const int row = idx / (C / 8), col = (idx % (C / 8)) * 8;
            *reinterpret_cast<u16x8*>(tg + row * C + col) = *reinterpret_cast<const u16x8*>(sT + row * TS + col);
        }
    }
}

// ====================================================================== single pass
template <int C, int DK, int VS>
struct DspLayout {
    using TK = SwzTile<DK>;     // K, and the hand-off rows of S_in
    using TV = SwzTile<VS>;     // the v slice, and the outputs waiting to be stored
    using TU = SwzTile<C>;      // the hand-off rows of U^T
    static constexpr int NV = VS / 16;
    static constexpr int TUS = C + 8;   // T_U rows 144 bytes apart: 8-byte row reads of 32 lanes on 64 banks
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    // gate tables of one chunk (floats): G, e^G, e^-G, carry weights e^(G_last - G), then
    // e^(G_last) and G_last
    static constexpr int GG = 0, GEG = C, GENG = 2 * C, GW = 3 * C, GEL = 4 * C, GL = 4 * C + 1;
    static constexpr int KBUF = al(C * TK::STRIDE * 2);
    static constexpr int VBUF = al(C * TV::STRIDE * 2);
    static constexpr int TBUF = al(C * TUS * 2);
    static constexpr int GBUF = al((4 * C + 4) * 4);
    static constexpr int HS = al(16 * TK::STRIDE * 2), HU = al(16 * TU::STRIDE * 2);
    static constexpr int HBUF = NV * (HS + 2 * HU);
    static constexpr int OBUF = VBUF;
    static constexpr int oK = 0;
    static constexpr int oV = oK + 3 * KBUF;
    static constexpr int oT = oV + 2 * VBUF;
    static constexpr int oG = oT + 2 * TBUF;
    static constexpr int oH = oG + 3 * GBUF;
    static constexpr int oO = oH + 2 * HBUF;
    static constexpr int bytes = oO + 2 * OBUF;
    static_assert(bytes <= 160 * 1024, "LDS budget of the delta single pass exceeded");
};

template <int C, int DK, int DV, int VS>
__global__ __launch_bounds__(256)
void delta_sp_kernel(DspParams p) {
    using Lay = DspLayout<C, DK, VS>;
    using TK = typename Lay::TK;
    using TV = typename Lay::TV;
    using TU = typename Lay::TU;
    constexpr int NT = 256;
    constexpr int NV = Lay::NV;
    constexpr int CT = C / 16, JB = CT / 2;     // token tiles, 32-token blocks
    constexpr int KT = DK / 16, KB = DK / 32;   // key tiles, 32-key blocks
    constexpr int TUS = Lay::TUS;
    static_assert(C == 64, "the output waves split four token tiles two by two");
    static_assert(DK >= 32 && DK % 32 == 0, "d_k in 32-key blocks");
    static_assert(DV % VS == 0 && (VS == 16 || VS == 32), "value slices of 16 or 32 channels");
    // staged pieces (16 bytes) of one chunk; ring index i holds one kind for every lane:
    // k (RK indices), the v slice (RV), T_U (RT), G (one index, 16 lanes: four floats each)
    constexpr int PK = C * DK / 8, PV = C * VS / 8, PT = C * C / 8, PG = C / 4;
    static_assert(PK % NT == 0 && PT % NT == 0 && PV <= NT && PG <= NT, "pieces per ring index");
    constexpr int RK = PK / NT, RV = 1, RT = PT / NT;
    constexpr int PER = RK + RV + RT + 1;
    constexpr int PO = C * VS / 8;   // 16-byte pieces of one chunk's outputs

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    auto sK = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oK + b * Lay::KBUF); };
    auto sV = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oV + b * Lay::VBUF); };
    auto sT = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oT + b * Lay::TBUF); };
    auto sG = [&](int b) { return reinterpret_cast<float*>(smem + Lay::oG + b * Lay::GBUF); };
    auto sO = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oO + b * Lay::OBUF); };
    auto hS = [&](int b, int vt) {
        return reinterpret_cast<u16*>(smem + Lay::oH + b * Lay::HBUF + vt * (Lay::HS + 2 * Lay::HU));
    };
    auto hUh = [&](int b, int vt) { return reinterpret_cast<u16*>(reinterpret_cast<unsigned char*>(hS(b, vt)) + Lay::HS); };
    auto hUl = [&](int b, int vt) {
        return reinterpret_cast<u16*>(reinterpret_cast<unsigned char*>(hS(b, vt)) + Lay::HS + Lay::HU);
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int lb = logical_block_of(blockIdx.x, gridDim.x, p.remap);
    const int bh = lb / p.slices, m0 = (lb % p.slices) * VS;
    const int T = p.T, NC = p.NC;
    const int64_t seq0 = static_cast<int64_t>(bh) * T;
    const int64_t seqk = static_cast<int64_t>(bh) * p.qk_seq;   // q and k rows
    const int64_t chunk0 = static_cast<int64_t>(bh) * NC;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    auto count = [&](int c) { return (T - c * C < C) ? (T - c * C) : C; };

    // Every wave issues the same global memory operations in the same order on every step -
    // the ring loads, its q rows, one 16-byte store of the outputs - so that the compiler's
    // count of operations in flight is exact on every path: each wait then covers only the
    // data it is for, and one step's loads stay in flight across the next step's work.

    // ---- register ring: the staged pieces of two chunks (indices clamped; consumed only
    // where they are written to LDS, just before a barrier)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 rg[2][PER];
    float rgl[2];
    auto load = [&](int c, u32x4 (&x)[PER], float& gl) {
        const int n = count(c);
        const int64_t t0 = static_cast<int64_t>(c) * C;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const void* src;
            if (i < RK) {
                const int q = tid + i * NT, j = q / (DK / 8), col = (q % (DK / 8)) * 8;
                src = p.k + (seqk + t0 + (j < n ? j : 0)) * DK + col;
            } else if (i < RK + RV) {
                const int e = tid < PV ? tid : 0, j = e / (VS / 8), col = (e % (VS / 8)) * 8;
                src = p.v + (seq0 + t0 + (j < n ? j : 0)) * DV + m0 + col;
            } else if (i < RK + RV + RT) {
                src = p.tu + (chunk0 + c) * C * C + (tid + (i - RK - RV) * NT) * 8;
            } else {
                src = p.g + (chunk0 + c) * C + (tid % PG) * 4;
            }
            x[i] = *reinterpret_cast<const u32x4*>(src);
        }
        gl = p.g[(chunk0 + c) * C + C - 1];
    };
    // chunk c into LDS slot set `slot` (K and the gate tables: slot % 3, the rest slot & 1)
    auto stage = [&](int c, int slot, const u32x4 (&x)[PER], float gl) {
        const int n = count(c);
        u16* K = sK(slot % 3);
        u16* V = sV(slot & 1);
        u16* TT = sT(slot & 1);
        float* GT = sG(slot % 3);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (i < RK) {
                const int q = tid + i * NT, j = q / (DK / 8), col = (q % (DK / 8)) * 8;
                *reinterpret_cast<u32x4*>(K + TK::off(j, col)) = j < n ? x[i] : __builtin_bit_cast(u32x4, z8);
            } else if (i < RK + RV) {
                const int j = tid / (VS / 8), col = (tid % (VS / 8)) * 8;
                if (tid < PV)
                    *reinterpret_cast<u32x4*>(V + TV::off(j, col)) = j < n ? x[i] : __builtin_bit_cast(u32x4, z8);
            } else if (i < RK + RV + RT) {
                const int e = tid + (i - RK - RV) * NT, row = e / (C / 8), col = (e % (C / 8)) * 8;
                *reinterpret_cast<u32x4*>(TT + row * TUS + col) = x[i];
            } else if (tid < PG) {
                const int j = tid * 4;
                const f32x4 G = __builtin_bit_cast(f32x4, x[i]);
                f32x4 eg, eng, wt;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    eg[e] = ex2(G[e]);
                    eng[e] = ex2(-G[e]);
                    wt[e] = ex2(gl - G[e]);
                }
                stf4(GT + Lay::GG + j, G);
                stf4(GT + Lay::GEG + j, eg);
                stf4(GT + Lay::GENG + j, eng);
                stf4(GT + Lay::GW + j, wt);
                if (j == 0) {
                    GT[Lay::GEL] = ex2(gl);
                    GT[Lay::GL] = gl;
                }
            }
        }
    };

    // ---- chain waves: S^T of value tile vt = w in fp32 accumulators,
    // sacc[ct][e] = S[m0 + 16 vt + r16][16 ct + 4g + e]
    const bool chain = w < NV;
    const bool outw = w >= 2;
    const int vt = chain ? w : 0;
    f32x4 sacc[KT];
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
        sacc[ct] = zf4();
        if (chain && p.s0 != nullptr)
            sacc[ct] = ldf4(p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * vt + r16) * DK + 16 * ct + 4 * g);
    }

    // ---- q rows of token tiles {0, 3} (waves 0 and 2) or {1, 2} (waves 1 and 3) in registers,
    // operand layout of the products over d_k (pieces rr_col); the output waves use them
    const int ow = w & 1;
    const int itA = ow == 0 ? 0 : 1, itB = ow == 0 ? 3 : 2;
    u16x8 qr[2][2][KB];
    auto load_q = [&](int c, u16x8 (&x)[2][KB]) {
        const int n = count(c);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int i = 16 * (s == 0 ? itA : itB) + r16;
            const int64_t row = seqk + static_cast<int64_t>(c) * C + (i < n ? i : 0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                x[s][kb] = *reinterpret_cast<const u16x8*>(p.q + row * DK + rr_col(kb, g, KB));
        }
    };
    // ---- the outputs of chunk c, from LDS to HBM: one 16-byte piece per thread
    auto store_o = [&](int c) {
        const int n = count(c);
        const u16* O = sO(c & 1);
        const int e = tid < PO ? tid : 0, j = e / (VS / 8), col = (e % (VS / 8)) * 8;
        const u16x8 x = *reinterpret_cast<const u16x8*>(O + TV::off(j, col));
        if (tid < PO && j < n)
            *reinterpret_cast<u16x8*>(p.o + (seq0 + static_cast<int64_t>(c) * C + j) * DV + m0 + col) = x;
    };

    // ---- one chunk of the chain (wave vt): Y, R, U, the hand-off and the carry
    auto chain_step = [&](int c) __attribute__((always_inline)) {
        const u16* K = sK(c % 3);
        const u16* V = sV(c & 1);
        const u16* TT = sT(c & 1);
        const float* GT = sG(c % 3);
        u16* HSo = hS(c & 1, vt);
        u16* HUh = hUh(c & 1, vt);
        u16* HUl = hUl(c & 1, vt);
        // S_in in bf16: the B operand of Y (reduction slots 32kb + 4g + e and 32kb + 16 + 4g + e)
        // and the rows handed to the output waves
        bf16x4 sb[KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            sb[ct] = cvt4(sacc[ct]);
            st4(HSo + TK::off(r16, 16 * ct + 4 * g), sb[ct]);
        }
        // Y = K S_in^T: y[it][e] = Y[16it + 4g + e][value r16]
        f32x4 y[CT];
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            f32x4 acc = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int row = 16 * it + r16;
                const bf16x8 a = join8(ld4(K + TK::off(row, 32 * kb + 4 * g)), ld4(K + TK::off(row, 32 * kb + 16 + 4 * g)));
                acc = mfma_16x16x32(a, join8(sb[2 * kb], sb[2 * kb + 1]), acc);
            }
            y[it] = acc;
        }
        // R = V - diag(e^G) Y, the B operand of U = T_U R (reduction slots 32jb + 4g + e and
        // 32jb + 16 + 4g + e)
        bf16x4 rb[CT];
#pragma unroll
        for (int jt = 0; jt < CT; ++jt) {
            const f32x4 v4 = up4(tr_op_s<VS>(V, 16 * jt, 16 * vt, r16, g));
            const f32x4 eg = ldf4(GT + Lay::GEG + 16 * jt + 4 * g);
            rb[jt] = cvt4(v4 - eg * y[jt]);
        }
        // U = T_U R (lower triangular: block jb reaches token tile it when 2jb <= it)
        f32x4 u[CT];
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            f32x4 acc = zf4();
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if (2 * jb > it) continue;
                const bool hi = 2 * jb + 1 <= it;
                const u16* tr = TT + (16 * it + r16) * TUS + 32 * jb + 4 * g;
                acc = mfma_16x16x32(join8(ld4(tr), hi ? ld4(tr + 16) : zero4()), join8(rb[2 * jb], rb[2 * jb + 1]), acc);
            }
            u[it] = acc;
        }
        // hand-off of U^T rows (bf16 hi + lo) for the output waves
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            const bf16x4 h = cvt4(u[it]);
            st4(HUh + TU::off(r16, 16 * it + 4 * g), h);
            st4(HUl + TU::off(r16, 16 * it + 4 * g), cvt4(u[it] - up4(h)));
        }
        // carry: S^T <- e^(G_last) S^T + K^T diag(e^(G_last - G)) U
        const float dec = GT[Lay::GEL];
        bf16x8 wb[JB];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
            wb[jb] = join8(cvt4(u[2 * jb] * ldf4(GT + Lay::GW + 32 * jb + 4 * g)),
                           cvt4(u[2 * jb + 1] * ldf4(GT + Lay::GW + 32 * jb + 16 + 4 * g)));
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            f32x4 acc = sacc[ct] * dec;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) acc = mfma_16x16x32(tr_split_s<DK>(K, jb, 16 * ct, true, r16, g), wb[jb], acc);
            sacc[ct] = acc;
        }
    };

    // ---- one chunk of the outputs (output wave): P for its two token tiles, then per value
    // tile o^T = S_in Q^T diag(e^G) + U^T P^T, written to the chunk's output buffer in LDS
    auto output_step = [&](int c, const u16x8 (&x)[2][KB]) __attribute__((always_inline)) {
        const u16* K = sK(c % 3);
        const float* GT = sG(c % 3);
        u16* O = sO(c & 1);
        const bool flat = GT[Lay::GL] >= -100.f;   // e^(G_i) e^(-G_j) both within 2^+-100
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int it = s == 0 ? itA : itB;
            const int i = 16 * it + r16;
            // P[i][16jt + 4g + e] = (q_i . k_j) e^(G_i - G_j), masked above the diagonal
            f32x4 pacc[CT];
#pragma unroll
            for (int jt = 0; jt < CT; ++jt) {
                pacc[jt] = zf4();
                if (jt > it) continue;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(K + TK::off(16 * jt + r16, rr_col(kb, g, KB)));
                    pacc[jt] = mfma_16x16x32(a, as_bf16x8(x[s][kb]), pacc[jt]);
                }
            }
            const float egi = GT[Lay::GEG + i];
            const float gi = GT[Lay::GG + i];
            bf16x4 pb[CT];
#pragma unroll
            for (int jt = 0; jt < CT; ++jt) {
                pb[jt] = zero4();
                if (jt > it) continue;
                f32x4 d;
                if (flat) {
                    d = ldf4(GT + Lay::GENG + 16 * jt + 4 * g) * egi;
                } else {
                    const f32x4 gj = ldf4(GT + Lay::GG + 16 * jt + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) d[e] = ex2(gi - gj[e]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * jt + 4 * g + e > i) d[e] = 0.f;
                pb[jt] = cvt4(pacc[jt] * d);
            }
#pragma unroll
            for (int t = 0; t < NV; ++t) {
                const u16* HSi = hS(c & 1, t);
                const u16* HUhi = hUh(c & 1, t);
                const u16* HUlo = hUl(c & 1, t);
                f32x4 acc = zf4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(HSi + TK::off(r16, rr_col(kb, g, KB)));
                    acc = mfma_16x16x32(a, as_bf16x8(x[s][kb]), acc);
                }
                acc = acc * egi;
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    if (2 * jb > it) continue;
                    const bool hi = 2 * jb + 1 <= it;
                    const bf16x8 pbb = join8(pb[2 * jb], pb[2 * jb + 1]);
                    const bf16x4 h0 = ld4(HUhi + TU::off(r16, 32 * jb + 4 * g));
                    const bf16x4 h1 = hi ? ld4(HUhi + TU::off(r16, 32 * jb + 16 + 4 * g)) : zero4();
                    const bf16x4 l0 = ld4(HUlo + TU::off(r16, 32 * jb + 4 * g));
                    const bf16x4 l1 = hi ? ld4(HUlo + TU::off(r16, 32 * jb + 16 + 4 * g)) : zero4();
                    acc = mfma_16x16x32(join8(h0, h1), pbb, acc);
                    acc = mfma_16x16x32(join8(l0, l1), pbb, acc);
                }
                // o[16it + r16][m0 + 16t + 4g + e]
                st4(O + TV::off(i, 16 * t + 4 * g), cvt4(acc));
            }
        }
    };

    // One step s (compile-time ring slot R = s & 1; STORE: s >= 2): the loads of chunk s + 2
    // and the q rows of chunk s, the store of chunk s - 2's outputs, the chain of chunk s, the
    // outputs of chunk s - 1, staging of chunk s + 1 into slot set s + 1 (past the end: a
    // copy of the last chunk, into slots no wave reads again: K slot s + 1 held chunk s - 2,
    // V and T_U slot s + 1 chunk s - 1).
    auto step = [&](int s, auto slot, auto with_store) __attribute__((always_inline)) {
        constexpr int R = decltype(slot)::value;
        load(s + 2 < NC ? s + 2 : NC - 1, rg[R], rgl[R]);
        load_q(s < NC ? s : NC - 1, qr[R]);
        if constexpr (decltype(with_store)::value) store_o(s - 2);
        if (chain && s < NC) chain_step(s);
        if (outw && s >= 1) output_step(s - 1, qr[R ^ 1]);
        stage(s + 1 < NC ? s + 1 : NC - 1, s + 1, rg[R ^ 1], rgl[R ^ 1]);
        lds_barrier();
    };

    if (NC > 0) {
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using NO = std::false_type;
        using YES = std::true_type;
        load(0, rg[0], rgl[0]);
        load(NC > 1 ? 1 : 0, rg[1], rgl[1]);
        stage(0, 0, rg[0], rgl[0]);
        lds_barrier();
        // steps 0 .. NC; the first two have no outputs to store yet
        step(0, I0{}, NO{});
        step(1, I1{}, NO{});
        int s = 2;
        for (; s + 1 <= NC; s += 2) {
            step(s, I0{}, YES{});
            step(s + 1, I1{}, YES{});
        }
        if (s <= NC) step(s, I0{}, YES{});
        // the last chunk's outputs (written by step NC)
        store_o(NC - 1);
    }

    if (chain && p.s_out != nullptr) {
        float* so = p.s_out + (static_cast<int64_t>(bh) * DV + m0 + 16 * vt + r16) * DK + 4 * g;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) stf4(so + 16 * ct, sacc[ct]);
    }
}

// ====================================================================== row norm
//
// DeltaNet's output norm ("Scrivere meglio nella memoria", section "Correggere: la delta
// rule": an RMS norm stabilises the readout): o <- o / sqrt(mean(o^2) + eps) * weight, in
// place on bf16 rows of DV channels, the sum of squares in fp32. A wave takes four rows, a
// row 16 lanes (DV / 16 channels each).
template <int DV>
__global__ __launch_bounds__(256)
void rms_rows_bf16_kernel(u16* o, const float* weight, float eps, int64_t rows) {
    constexpr int PER = DV / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t row = (static_cast<int64_t>(blockIdx.x) * 256 + tid) / 16;
    const int part = lane & 15;
    const bool live = row < rows;
    u16* r = o + (live ? row : 0) * DV + part * PER;
    float x[PER];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        x[e] = bf16_bits_to_f32(r[e]);
        ss += x[e] * x[e];
    }
    ss = row16_sum(ss);
    const float inv = 1.f / __builtin_sqrtf(ss / static_cast<float>(DV) + eps);
    if (live) {
#pragma unroll
        for (int e = 0; e < PER; ++e) r[e] = f32_to_bf16_bits(x[e] * inv * weight[part * PER + e]);
    }
}

// ====================================================================== launch
template <int C, int DK, int DV>
hipError_t launch_dsp_dv(const ChunkArgs& a, hipStream_t stream) {
    constexpr int VS = DV >= 32 ? 32 : 16;
    const int NC = (a.T + C - 1) / C;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    DspParams p;
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.alpha = a.gate;
    p.beta = a.beta;
    p.s0 = a.s0;
    p.o = static_cast<u16*>(a.o);
    p.s_out = a.s_out;
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    const int64_t chunks = heads * NC;
    p.tu = reinterpret_cast<u16*>(ws);
    ws += delta_ws_align(chunks * C * C * 2);
    p.g = reinterpret_cast<float*>(ws);
    ws += delta_ws_align(chunks * C * 4);
    p.map = (a.fuse & 1) ? 1 : 0;
    p.qraw = p.q;
    p.kraw = p.k;
    p.kmap = reinterpret_cast<u16*>(ws);
    p.qmap = reinterpret_cast<u16*>(ws + delta_ws_align(chunks * C * DK * 2));
    if (p.map) {
        // the mapped copies are [BH * NC][C][DK]: the token-major layout of q and k with rows
        // padded to whole chunks, read by the single pass through per-sequence offsets
        p.k = p.kmap;
        p.q = p.qmap;
    }
    p.T = a.T;
    p.NC = NC;
    p.qk_seq = p.map ? NC * C : a.T;
    p.slices = DV / VS;
    const int64_t grid = heads * p.slices;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    if (NC > 0) {
        hipLaunchKernelGGL((delta_tfac_kernel<C, DK>), dim3(static_cast<unsigned>(heads * NC)), dim3(256), 0, stream, p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((delta_sp_kernel<C, DK, DV, VS>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || !(a.fuse & 2)) return err;
    const int64_t rows = heads * a.T;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL((rms_rows_bf16_kernel<DV>), dim3(static_cast<unsigned>((rows * 16 + 255) / 256)), dim3(256), 0,
                       stream, static_cast<u16*>(a.o), a.onw, a.oeps, rows);
    return hipGetLastError();
}

template <int C, int DK>
hipError_t launch_dsp_dk(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_dsp_dv<C, DK, 16>(a, stream);
        case 32: return launch_dsp_dv<C, DK, 32>(a, stream);
        case 64: return launch_dsp_dv<C, DK, 64>(a, stream);
        case 128: return launch_dsp_dv<C, DK, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int C>
hipError_t launch_dsp(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 32: return launch_dsp_dk<C, 32>(a, stream);
        case 64: return launch_dsp_dk<C, 64>(a, stream);
        case 128: return launch_dsp_dk<C, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
