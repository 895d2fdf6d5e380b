// Chunkwise forward with bfloat16 storage: bf16 MFMA (v_mfma_f32_16x16x32_bf16
// and 16x16x16) for the contractions, fp32 accumulation, fp32 memory in registers.
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
// Work decomposition (gfx950). Gates act on key channels (columns of S), so
// rows of S (value channels) evolve independently: a workgroup owns one
// (batch, head) and DVT = 16 * MT value channels; several workgroups share a
// head when that is needed to occupy the 256 CUs. Inside the workgroup,
// MT * KS waves split the workgroup's slice of S^T by value-channel tile (mt)
// and key-channel range (ks): each wave keeps its d_k/KS x 16 block of S^T in
// MFMA accumulators for the whole sequence. Per chunk:
//   staging   q, k, v (and gates) of chunk c+1 are fetched from HBM into
//             registers while chunk c computes (16-byte coalesced loads), then
//             written to LDS in the layouts the MFMA operands need (token-major
//             q, k; channel-major k^T and v^T with the carry weights folded in);
//             every wave also publishes its block of S^T in bf16;
//   phase 1   the S-independent triangle: P (and the delta rule's A) tiles,
//             spread over all waves, written to LDS;
//   (delta)   T's 16x16 diagonal blocks by forward substitution, then W and U0
//             by blocked forward substitution on MFMA; U = U0 - W S^T per
//             token tile, shared through LDS in fp32;
//   outputs   each wave finishes the 16-token row tiles it owns: P V (or P U)
//             plus the readout of the incoming memory over the full d_k;
//             results leave through LDS as 16-byte stores;
//   carry     each wave updates its own block of S^T (K^T V, or K^T U).
// MFMA k-slots use the "split" assignment: within a 32-wide reduction block,
// lane (r, g) feeds indices 4g..4g+3 of the block's first 16 and 4g..4g+3 of
// its second 16 - exactly the rows a 16x16 accumulator tile holds per lane, so
// accumulator tiles feed later products directly.
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

// Operand from a row-major LDS array X (row stride RS elements) for reduction block kb:
// split k-slots, the second half zero when the reduction has only 2*kb+1 tiles.
template <int NTILE, int RS>
__device__ __forceinline__ bf16x8 split_op(const u16* X, int row, int kb, int g) {
    const u16* p = X + row * RS + 32 * kb + 4 * g;
    return join8(ld4(p), (2 * kb + 1 < NTILE) ? ld4(p + 16) : zero4());
}

// LDS layout (bytes) of one kernel configuration.
template <int VARIANT, int C, int DK, int MT, int KS>
struct Layout {
    static constexpr int NW = MT * KS;
    static constexpr int DVT = 16 * MT;
    static constexpr int CT = C / 16;
    static constexpr int QS = DK + 8;   // token-major bf16 row stride
    static constexpr int TS = C + 8;    // score-tile (P) bf16 row stride
    static constexpr int AS = C + 4;    // fp32 triangular-system row stride
    static constexpr int BS = DK + 4;   // fp32 cumulative-gate row stride
    static constexpr int SS = DK + 8;   // bf16 S^T row stride (one row per value channel)
    static constexpr int US = C + 4;    // fp32 U row stride (one row per value channel)
    static constexpr int OS = 24;       // output staging row stride (u16)
    static constexpr bool kGla = VARIANT == kGLA;
    static constexpr bool kDel = VARIANT == kGDelta;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int VS = DVT + 8;  // token-major v tile row stride
    static constexpr int oQ = 0;
    static constexpr int oK = al(oQ + C * QS * 2);
    static constexpr int oKw = al(oK + C * QS * 2);
    static constexpr int oV = al(oKw + (kDel ? 0 : C * QS * 2));
    static constexpr int oP = al(oV + C * VS * 2);
    static constexpr int oS = al(oP + C * TS * 2);
    static constexpr int oO = al(oS + DVT * SS * 2);
    static constexpr int oG = al(oO + NW * 16 * OS * 2);
    static constexpr int oBeta = al(oG + (C + 1) * 4);
    static constexpr int oExtra = al(oBeta + C * 4);
    // GLA: rescaled q e^b, cumulative gates, factor tables
    static constexpr int oQe = oExtra;
    static constexpr int oB = al(oQe + (kGla ? C * QS * 2 : 0));
    static constexpr int oTab = al(oB + (kGla ? C * BS * 4 : 0));
    static constexpr int endGla = al(oTab + (kGla ? (CT * CT + 2 * CT + 1) * DK * 4 : 0));
    // delta rule: triangular system, diagonal inverses, W, shared U
    static constexpr int oA = oExtra;
    static constexpr int oD = al(oA + (kDel ? C * AS * 4 : 0));
    static constexpr int oW = al(oD + (kDel ? CT * 256 * 4 : 0));
    static constexpr int endW = al(oW + (kDel ? C * QS * 2 : 0));
    // U overlays q (dead once the incoming-memory readout is done) when it fits
    static constexpr bool kUoverlay = DVT * US * 4 <= C * QS * 2;
    static constexpr int oU = kUoverlay ? oQ : endW;
    static constexpr int endDel = kUoverlay ? endW : al(endW + (kDel ? DVT * US * 4 : 0));
    static constexpr int bytes = kGla ? endGla : (kDel ? endDel : oExtra);
    static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
};

template <int VARIANT, int C, int DK, int MT, int KS>
__global__ __launch_bounds__(64 * MT * KS)
void chunk_kernel(Params p) {
    using Lay = Layout<VARIANT, C, DK, MT, KS>;
    constexpr int NW = MT * KS;
    constexpr int NT = 64 * NW;
    constexpr int DVT = 16 * MT;
    constexpr int CT = C / 16;           // 16-token tiles per chunk
    constexpr int KT = DK / 16;          // 16-channel tiles of the key dimension
    static_assert(KT % KS == 0, "key split must divide the key tiles");
    constexpr int KTW = KT / KS;         // key tiles owned by one wave
    constexpr int KB = (KT + 1) / 2;     // 32-wide reduction blocks over d_k
    constexpr int JB = (CT + 1) / 2;     // 32-wide reduction blocks over the chunk
    constexpr int QS = Lay::QS, TS = Lay::TS, AS = Lay::AS, BS = Lay::BS, VS = Lay::VS;
    constexpr int SS = Lay::SS, US = Lay::US, OS = Lay::OS;
    constexpr bool kGla = Lay::kGla;
    constexpr bool kDel = Lay::kDel;

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sQ = reinterpret_cast<u16*>(smem + Lay::oQ);
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    // carry-weighted k (the delta rule weights U instead and carries with raw k)
    u16* const sKw = kDel ? reinterpret_cast<u16*>(smem + Lay::oK) : reinterpret_cast<u16*>(smem + Lay::oKw);
    u16* const sV = reinterpret_cast<u16*>(smem + Lay::oV);
    u16* const sP = reinterpret_cast<u16*>(smem + Lay::oP);
    u16* const sS = reinterpret_cast<u16*>(smem + Lay::oS);
    u16* const sO = reinterpret_cast<u16*>(smem + Lay::oO);
    float* const sG = reinterpret_cast<float*>(smem + Lay::oG);      // retention: g^k table; delta: G
    float* const sBeta = reinterpret_cast<float*>(smem + Lay::oBeta);
    u16* const sQe = reinterpret_cast<u16*>(smem + Lay::oQe);
    float* const sB = reinterpret_cast<float*>(smem + Lay::oB);
    float* const tabF = reinterpret_cast<float*>(smem + Lay::oTab);
    float* const tabZ = tabF + CT * CT * DK;
    float* const tabL = tabZ + CT * DK;
    float* const tabDec = tabL + CT * DK;
    float* const sA = reinterpret_cast<float*>(smem + Lay::oA);
    float* const sD = reinterpret_cast<float*>(smem + Lay::oD);
    u16* const sW = reinterpret_cast<u16*>(smem + Lay::oW);
    float* const sU = reinterpret_cast<float*>(smem + Lay::oU);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mt = w % MT;               // value-channel tile of this wave
    const int ks = w / MT;               // key-channel range of this wave
    const int ct0 = ks * KTW;            // first key tile of this wave
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

    // retention: log2 of the head's decay, and this lane's output scales g^(i+1) for the
    // rows i = 16it + 4g + r it finishes (the same for every full chunk)
    const float lg2 = (VARIANT == kRetention) ? p.gate[h] * kLog2e : 0.f;
    f32x4 oscale[VARIANT == kRetention ? CT : 1];
    if constexpr (VARIANT == kRetention) {
#pragma unroll
        for (int it = 0; it < CT; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r) oscale[it][r] = ex2(static_cast<float>(16 * it + 4 * g + r + 1) * lg2);
    }

    // ---- this wave's block of the memory: sacc[t][r] = S[v0 + 16mt + r16][16(ct0+t) + 4g + r]
    f32x4 sacc[KTW];
    {
        const float* srow = p.s0 ? p.s0 + (static_cast<int64_t>(bh) * dv + v0 + 16 * mt + r16) * DK : nullptr;
#pragma unroll
        for (int t = 0; t < KTW; ++t) sacc[t] = srow ? ldf4(srow + 16 * (ct0 + t) + 4 * g) : zf4();
    }

    // ---- register staging of one chunk: 4-row micro-tiles of QV columns (16- or 8-byte
    // loads; 8-byte ones when that is what it takes to give every thread a tile)
    constexpr int QV = ((C / 4) * (DK / 8) >= NT) ? 8 : 4;
    typedef typename Vec<QV>::type qv_t;
    constexpr int QK_ITEMS = (C / 4) * (DK / QV);
    constexpr int QK_PER = (QK_ITEMS + NT - 1) / NT;
    constexpr int V_ITEMS = (C / 4) * (DVT / 8);
    constexpr int V_PER = (V_ITEMS + NT - 1) / NT;
    constexpr int G_ITEMS = kGla ? (C / 4) * (DK / 4) : 0;
    constexpr int G_PER = kGla ? (G_ITEMS + NT - 1) / NT : 1;
    qv_t rq[QK_PER][4], rk[QK_PER][4];
    u16x8 rv[V_PER][4];
    f32x4 rg[G_PER][4];
    float rla = 0.f, rbe = 0.f;

    // Chunk base pointers are uniform (scalar registers); per-lane offsets stay 32-bit.
    auto fetch = [&](int t0, int n) {
        const u16* qc = qg + static_cast<int64_t>(t0) * DK;
        const u16* kc = kg + static_cast<int64_t>(t0) * DK;
        const u16* vc = vg + static_cast<int64_t>(t0) * dv;
#pragma unroll
        for (int pi = 0; pi < QK_PER; ++pi) {
            const int item = tid + pi * NT;
            if (item < QK_ITEMS) {
                const int row0 = (item / (DK / QV)) * 4, col0 = (item % (DK / QV)) * QV;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const bool in = row0 + rr < n;
                    const unsigned off = static_cast<unsigned>((row0 + rr) * DK + col0);
                    qv_t z = {};
                    rq[pi][rr] = in ? *reinterpret_cast<const qv_t*>(qc + off) : z;
                    rk[pi][rr] = in ? *reinterpret_cast<const qv_t*>(kc + off) : z;
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
                        ? *reinterpret_cast<const u16x8*>(vc + static_cast<unsigned>((row0 + rr) * dv + col0))
                        : z;
                }
            }
        }
        if constexpr (kGla) {
            const float* gc = p.gate + (tok0 + t0) * DK;
#pragma unroll
            for (int pi = 0; pi < G_PER; ++pi) {
                const int item = tid + pi * NT;
                if (item < G_ITEMS) {
                    const int row0 = (item / (DK / 4)) * 4, col0 = (item % (DK / 4)) * 4;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        rg[pi][rr] = (row0 + rr < n) ? ldf4(gc + static_cast<unsigned>((row0 + rr) * DK + col0))
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

    const int n_chunks = (T + C - 1) / C;
    if (n_chunks > 0) fetch(0, T < C ? T : C);

    for (int ch = 0; ch < n_chunks; ++ch) {
        const int t0 = ch * C;
        const int n = (T - t0 < C) ? (T - t0) : C;
        lds_barrier();  // every wave is done with the previous chunk's LDS

        // ------------------------------------------------------------ staging
        // the wave's block of S^T, bf16, one row per value channel
#pragma unroll
        for (int t = 0; t < KTW; ++t) st4(sS + (16 * mt + r16) * SS + 16 * (ct0 + t) + 4 * g, cvt4(sacc[t]));
        // v tile (raw, token-major)
#pragma unroll
        for (int pi = 0; pi < V_PER; ++pi) {
            const int item = tid + pi * NT;
            if (item < V_ITEMS) {
                const int row0 = (item / (DVT / 8)) * 4, col0 = (item % (DVT / 8)) * 8;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<u16x8*>(sV + (row0 + rr) * VS + col0) = rv[pi][rr];
            }
        }
        if constexpr (!kGla) {
#pragma unroll
            for (int pi = 0; pi < QK_PER; ++pi) {
                const int item = tid + pi * NT;
                if (item < QK_ITEMS) {
                    const int row0 = (item / (DK / QV)) * 4, col0 = (item % (DK / QV)) * QV;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        *reinterpret_cast<qv_t*>(sQ + (row0 + rr) * QS + col0) = rq[pi][rr];
                        *reinterpret_cast<qv_t*>(sK + (row0 + rr) * QS + col0) = rk[pi][rr];
                    }
                    if constexpr (VARIANT == kRetention) {
                        // the carry weight g^(n-1-j) folded into a second copy of k
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int j = row0 + rr;
                            const float wgt = (j < n) ? ex2(static_cast<float>(n - 1 - j) * lg2) : 0.f;
                            qv_t t;
#pragma unroll
                            for (int e = 0; e < QV; ++e)
                                t[e] = bits(static_cast<__bf16>(bf16_bits_to_f32(rk[pi][rr][e]) * wgt));
                            *reinterpret_cast<qv_t*>(sKw + j * QS + col0) = t;
                        }
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
                    for (int rr = 0; rr < 4; ++rr) stf4(sB + (row0 + rr) * BS + col0, rg[pi][rr] * kLog2e);
                }
            }
            lds_barrier();
            for (int c = w; c < DK; c += NW) {
                float x = (lane < C) ? sB[lane * BS + c] : 0.f;
                x = wave_inclusive_scan(x);
                if (lane < C) sB[lane * BS + c] = x;
            }
            lds_barrier();
            // factor tables per key channel; the reference point of token tile t is the
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
            lds_barrier();
            // q rescaled to its tile's reference, q e^b, k rescaled, carry-weighted k^T
#pragma unroll
            for (int pi = 0; pi < QK_PER; ++pi) {
                const int item = tid + pi * NT;
                if (item < QK_ITEMS) {
                    const int row0 = (item / (DK / QV)) * 4, col0 = (item % (DK / QV)) * QV;
                    const int t = row0 / 16;
                    float ref[QV], zf[QV], lf[QV];
#pragma unroll
                    for (int e = 0; e < QV; ++e) {
                        ref[e] = (t == 0) ? 0.f : sB[(16 * t - 1) * BS + col0 + e];
                        zf[e] = tabZ[t * DK + col0 + e];
                        lf[e] = tabL[t * DK + col0 + e];
                    }
                    float kd[4][QV];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int i = row0 + rr;
                        qv_t oq, oqe, ok;
#pragma unroll
                        for (int e = 0; e < QV; ++e) {
                            const float b = sB[i * BS + col0 + e];
                            const float E = ex2(b - ref[e]);
                            const float Ei = ex2(ref[e] - b);
                            const float qx = bf16_bits_to_f32(rq[pi][rr][e]) * E;
                            kd[rr][e] = bf16_bits_to_f32(rk[pi][rr][e]) * Ei;
                            oq[e] = bits(static_cast<__bf16>(qx));
                            oqe[e] = bits(static_cast<__bf16>(qx * zf[e]));
                            ok[e] = bits(static_cast<__bf16>(kd[rr][e]));
                        }
                        *reinterpret_cast<qv_t*>(sQ + i * QS + col0) = oq;
                        *reinterpret_cast<qv_t*>(sQe + i * QS + col0) = oqe;
                        *reinterpret_cast<qv_t*>(sK + i * QS + col0) = ok;
                        qv_t okw;
#pragma unroll
                        for (int e = 0; e < QV; ++e) okw[e] = bits(static_cast<__bf16>(kd[rr][e] * lf[e]));
                        *reinterpret_cast<qv_t*>(sKw + i * QS + col0) = okw;
                    }
                }
            }
        }
        lds_barrier();

        // chunk ch is in LDS: fetch the next one while this one computes
        if (ch + 1 < n_chunks) {
            const int t1 = t0 + C;
            fetch(t1, (T - t1 < C) ? (T - t1) : C);
        }

        // ------------------------------------------------------------ phase 1: the triangle
        constexpr int NPAIR = CT * (CT + 1) / 2;
        constexpr int NQ = (NPAIR + NW - 1) / NW;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
            const int pr = w + NW * qq;            // pairs (it, jt), jt <= it, in row order
            if (pr < NPAIR) {
                int it = 0, jt = pr;
                while (jt > it) { jt -= it + 1; ++it; }
                const int i = 16 * it + r16;
                // operands of the delta rule's decay and write strength, loaded up front
                float gi = 0.f, bi = 0.f;
                f32x4 gj = zf4();
                if constexpr (kDel) {
                    gi = sG[i];
                    bi = sBeta[i];
                    gj = ldf4(sG + 16 * jt + 4 * g);
                }
                f32x4 acc = zf4(), acc2 = zf4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 a = split_op<KT, QS>(sK, 16 * jt + r16, kb, g);
                    bf16x8 bq = split_op<KT, QS>(sQ, i, kb, g);
                    if constexpr (kGla) {
                        if (jt < it) {
                            const float* F = tabF + (it * CT + jt) * DK + 32 * kb + 4 * g;
                            const f32x4 flo = ldf4(F);
                            const f32x4 fhi = (2 * kb + 1 < KT) ? ldf4(F + 16) : zf4();
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                bq[e] = static_cast<__bf16>(static_cast<float>(bq[e]) * flo[e]);
                                bq[4 + e] = static_cast<__bf16>(static_cast<float>(bq[4 + e]) * fhi[e]);
                            }
                        }
                    }
                    acc = mfma_16x16x32(a, bq, acc);
                    if constexpr (kDel) acc2 = mfma_16x16x32(a, split_op<KT, QS>(sK, i, kb, g), acc2);
                }
                // acc[r] = sum_c k[j][c] q[i][c] with j = 16jt + 4g + r, i = 16it + r16
                bf16x4 pv;
                f32x4 av;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jt + 4 * g + r;
                    float val, aval = 0.f;
                    if constexpr (VARIANT == kRetention) {
                        val = acc[r] * ex2(static_cast<float>(i - j) * lg2);
                    } else if constexpr (kGla) {
                        val = acc[r];
                    } else {
                        const float gam = ex2(fminf(gi - gj[r], 0.f));
                        val = acc[r] * gam;
                        aval = (j < i) ? bi * acc2[r] * gam : 0.f;
                    }
                    pv[r] = static_cast<__bf16>((j <= i) ? val : 0.f);
                    av[r] = aval;
                }
                st4(sP + i * TS + 16 * jt + 4 * g, pv);
                if constexpr (kDel) stf4(sA + i * AS + 16 * jt + 4 * g, av);
            }
        }
        lds_barrier();

        // incoming-memory readout over the full d_k for the row tiles this wave owns
        // (tile it belongs to key range it % KS), from the published bf16 S^T
        const u16* qsrc = kGla ? sQe : sQ;
        const u16* srow = sS + (16 * mt + r16) * SS;
        f32x4 oe[CT];
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            oe[it] = zf4();
            if (it % KS == ks) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const bf16x8 sb = join8(ld4(srow + 32 * kb + 4 * g),
                                            (2 * kb + 1 < KT) ? ld4(srow + 32 * kb + 16 + 4 * g) : zero4());
                    oe[it] = mfma_16x16x32(split_op<KT, QS>(qsrc, 16 * it + r16, kb, g), sb, oe[it]);
                }
            }
        }

        // U (delta rule): this wave's copy for all token tiles, fp32; output scales e^(G_i)
        f32x4 U[kDel ? CT : 1];
        f32x4 gscale[kDel ? CT : 1];
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
            lds_barrier();
            // ---------------------------------------------------- blocked forward substitution
            // X_b = D_b (R_b - sum_{kk<b} A_{b,kk} X_kk) for the right-hand sides
            // diag(beta e^G) K (-> W, LDS) and diag(beta) V (-> U0, registers)
            auto solve = [&](auto rhs, f32x4 (&X)[CT]) {
#pragma unroll
                for (int b = 0; b < CT; ++b) {
                    f32x4 acc = rhs(b);
#pragma unroll
                    for (int kk = 0; kk < b; ++kk) {
                        const f32x4 a = ldf4(sA + (16 * b + r16) * AS + 16 * kk + 4 * g);
                        acc = mfma16k(cvt4(-a), cvt4(X[kk]), acc);
                    }
                    const f32x4 d = ldf4(sD + b * 256 + r16 * 16 + 4 * g);
                    X[b] = mfma16k(cvt4(d), cvt4(acc), zf4());
                }
            };
            for (int nt = w; nt < KT; nt += NW) {
                f32x4 X[CT];
                solve([&](int b) {
                    const bf16x4 kv = tr_op<QS>(sK, 16 * b, 16 * nt, r16, g);
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
                const bf16x4 vv = tr_op<VS>(sV, 16 * b, 16 * mt, r16, g);
                f32x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = static_cast<float>(vv[e]) * sBeta[16 * b + 4 * g + e];
                return r;
            }, U);
            lds_barrier();
            // ---------------------------------------------------- U = U0 - W S^T, the token tiles
            // this wave owns (tile b belongs to key range b % KS), published in fp32
#pragma unroll
            for (int b = 0; b < CT; ++b) {
                if (b % KS == ks) {
                    f32x4 x = zf4();
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const bf16x8 sb = join8(ld4(srow + 32 * kb + 4 * g),
                                                (2 * kb + 1 < KT) ? ld4(srow + 32 * kb + 16 + 4 * g) : zero4());
                        x = mfma_16x16x32(split_op<KT, QS>(sW, 16 * b + r16, kb, g), sb, x);
                    }
                    stf4(sU + (16 * mt + r16) * US + 16 * b + 4 * g, U[b] - x);
                }
            }
            lds_barrier();
#pragma unroll
            for (int b = 0; b < CT; ++b) U[b] = ldf4(sU + (16 * mt + r16) * US + 16 * b + 4 * g);
#pragma unroll
            for (int it = 0; it < CT; ++it) {
                const f32x4 gv = ldf4(sG + 16 * it + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) gscale[it][r] = ex2(gv[r]);
            }
        }

        // ------------------------------------------------------------ outputs of the owned row tiles
        u16* const so = sO + w * 16 * OS;
        u16* const oc = og + static_cast<int64_t>(t0) * dv;
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            if (it % KS != ks) continue;
            f32x4 oi = zf4();
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if (2 * jb <= it) {
                    const bool hi = 2 * jb + 1 <= it;
                    const u16* prow = sP + (16 * it + r16) * TS + 32 * jb + 4 * g;
                    const bf16x8 a = join8(ld4(prow), hi ? ld4(prow + 16) : zero4());
                    if constexpr (kDel) {
                        // U enters as a bf16 hi + lo pair: its rounding would otherwise be the
                        // dominant error of the output
                        const f32x4 u0 = U[2 * jb];
                        const f32x4 u1 = hi ? U[2 * jb + 1] : zf4();
                        const bf16x4 h0 = cvt4(u0), h1 = cvt4(u1);
                        oi = mfma_16x16x32(a, join8(h0, h1), oi);
                        oi = mfma_16x16x32(a, join8(cvt4(u0 - up4(h0)), cvt4(u1 - up4(h1))), oi);
                    } else {
                        const bf16x4 vlo = tr_op<VS>(sV, 32 * jb, 16 * mt, r16, g);
                        const bf16x4 vhi = hi ? tr_op<VS>(sV, 32 * jb + 16, 16 * mt, r16, g) : zero4();
                        oi = mfma_16x16x32(a, join8(vlo, vhi), oi);
                    }
                }
            }
            f32x4 scale;
            if constexpr (VARIANT == kRetention) scale = oscale[it];
            else if constexpr (kDel) scale = gscale[it];
            else scale = f32x4{1.f, 1.f, 1.f, 1.f};
            bf16x4 res;
#pragma unroll
            for (int r = 0; r < 4; ++r) res[r] = static_cast<__bf16>(oi[r] + scale[r] * oe[it][r]);
            // 16 x 16 tile -> LDS -> one 16-byte store per half row
#pragma unroll
            for (int r = 0; r < 4; ++r) so[(4 * g + r) * OS + r16] = bits(res[r]);
            if (lane < 32) {
                const int row = lane >> 1, half = lane & 1;
                const u16x8 val = *reinterpret_cast<const u16x8*>(so + row * OS + 8 * half);
                if (16 * it + row < n)
                    *reinterpret_cast<u16x8*>(oc + static_cast<unsigned>((16 * it + row) * dv + 16 * mt + 8 * half)) = val;
            }
        }

        // ------------------------------------------------------------ memory carried on (own key tiles)
        float dec_s = 1.f;
        if constexpr (VARIANT == kRetention) dec_s = ex2(static_cast<float>(n) * lg2);
        float glast = 0.f;
        f32x4 wU[kDel ? CT : 1];
        if constexpr (kDel) {
            glast = sG[C - 1];   // padded tail tokens have log-gate 0
            dec_s = ex2(glast);
#pragma unroll
            for (int b = 0; b < CT; ++b) {
                const f32x4 gv = ldf4(sG + 16 * b + 4 * g);
#pragma unroll
                for (int e = 0; e < 4; ++e) wU[b][e] = U[b][e] * ex2(glast - gv[e]);
            }
        }
#pragma unroll
        for (int t = 0; t < KTW; ++t) {
            const int ct = ct0 + t;
            f32x4 acc;
            if constexpr (kGla) acc = sacc[t] * ldf4(tabDec + 16 * ct + 4 * g);
            else acc = sacc[t] * dec_s;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                const bool hi = 2 * jb + 1 < CT;
                const bf16x8 a = join8(tr_op<QS>(sKw, 32 * jb, 16 * ct, r16, g),
                                       hi ? tr_op<QS>(sKw, 32 * jb + 16, 16 * ct, r16, g) : zero4());
                if constexpr (kDel) {
                    acc = mfma_16x16x32(a, join8(cvt4(wU[2 * jb]), hi ? cvt4(wU[2 * jb + 1]) : zero4()), acc);
                } else {
                    const bf16x8 b = join8(tr_op<VS>(sV, 32 * jb, 16 * mt, r16, g),
                                           hi ? tr_op<VS>(sV, 32 * jb + 16, 16 * mt, r16, g) : zero4());
                    acc = mfma_16x16x32(a, b, acc);
                }
            }
            sacc[t] = acc;
        }
    }

    if (p.s_out) {
        float* srow = p.s_out + (static_cast<int64_t>(bh) * dv + v0 + 16 * mt + r16) * DK;
#pragma unroll
        for (int t = 0; t < KTW; ++t) stf4(srow + 16 * (ct0 + t) + 4 * g, sacc[t]);
    }
}

template <int VARIANT, int C, int DK, int MT, int KS>
hipError_t launch_cfg(const ChunkArgs& a, hipStream_t stream) {
    constexpr int DVT = 16 * MT;
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
    hipLaunchKernelGGL((chunk_kernel<VARIANT, C, DK, MT, KS>), dim3(static_cast<unsigned>(G)), dim3(64 * MT * KS),
                       0, stream, p);
    return hipGetLastError();
}

// Workgroup shape: the widest value-channel tile (MT * 16) that still gives every
// CU a workgroup, then split the key dimension over KS waves per value tile so a
// workgroup has up to 8 waves (two per SIMD, to hide each other's latencies).
constexpr int kCUs = 256;

template <int VARIANT, int C, int DK, int MT>
hipError_t launch_mt(const ChunkArgs& a, hipStream_t stream) {
    constexpr int KT = DK / 16;
    constexpr int KS = (KT < 8 / MT) ? KT : 8 / MT;
    return launch_cfg<VARIANT, C, DK, MT, KS>(a, stream);
}

template <int VARIANT, int C, int DK>
hipError_t launch_dk(const ChunkArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    int mt = 1;
    for (int cand = 4; cand >= 1; cand >>= 1) {
        if (16 * cand <= a.dv && heads * (a.dv / (16 * cand)) >= kCUs) { mt = cand; break; }
    }
    switch (mt) {
        case 4: return launch_mt<VARIANT, C, DK, 4>(a, stream);
        case 2: return launch_mt<VARIANT, C, DK, 2>(a, stream);
        default: return launch_mt<VARIANT, C, DK, 1>(a, stream);
    }
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
