// Gated delta rule, chunk 64, bf16 storage: a chunk-parallel prep and a single pass that
// keeps the memory on chip (the same single pass also serves retention and the scalar decay).
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
//   single pass  (chunks in order) one workgroup per (sequence, VS value channels);
//   row norm     (with DeltaNet's output norm fused in) every output row RMS-normalised in
//                place, one wave per four rows.
//
// Single pass, four waves. Rows of S (value channels) evolve independently, so waves 0 and 1
// (the "chain" waves) own 16 (or, without the delta step, 32) value channels each and keep
// S^T for them (every key) in fp32 MFMA accumulators; each product of the chain takes the
// previous one's accumulators directly as its B operand (bf16, a fixed permutation of the
// reduction slots), with nothing exchanged between waves:
//   Y = K S_in^T           (reduction over keys; K rows from LDS)
//   R = V - diag(e^G) Y,   U = T_U R    (reduction over tokens; T_U rows from LDS)
//   o^T = S_in Q^T diag(e^G) + U^T P^T  (U as a bf16 hi + lo pair)
//   S^T <- e^(G_last) S^T + K^T diag(e^(G_last - G)) U    (K^T by ds_read_b64_tr_b16)
// Waves 2 and 3 (the "helper" waves) issue every global load: K, Q, the v slice, T_U and G
// two chunks ahead into a register ring, written to LDS just before the chunk's barrier; and
// they form the decayed triangle P = (Q K^T . Gamma) masked one chunk ahead of the chain
// (token tiles {0, 3} and {1, 2}: five 16 x 16 tiles each; with one live chain wave, at
// 16-channel slices, the other chain wave forms tiles {0, 1} and the helpers {3} and {2}).
// K, Q and the gate tables live in three LDS slots (staged, the triangle's chunk, the chain's
// chunk), the rest in two. One workgroup barrier per chunk. The value slices of one sequence
// get block ids on one XCD and share its L2 copy of K, Q and T_U.
//
// Without the delta step (U = V: retention, "RetNet: la retention e le sue tre forme", and
// the scalar data-dependent decay, "Scrivere meglio nella memoria", section "Dimenticare: i
// gate") the same pass runs with no prep: the helpers form G from log gamma, or scan the raw
// log alpha, when they stage a chunk; Y, R and T_U drop out, and P V needs no lo part (V is
// exact in bf16). A chain wave may then carry two value tiles, so that one read of its K, Q
// and P operands serves 32 channels.
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

// The single pass's buffer offsets are 31-bit: one sequence's q, k, v or o (rows padded to
// whole chunks) must stay below 2^31 bytes.
inline bool delta_sp_fits(int T, int dk, int dv) {
    const long long rows = (static_cast<long long>(T) + 63) / 64 * 64;
    const long long d = dk > dv ? dk : dv;
    return dk >= 32 && rows * (d > 64 ? d : 64) * 2 < (1ll << 31);
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
    u16* tfull;           // [BH * NC][C][C] T = (I + A)^-1 itself (the backward's), or null
    // feature map fused in: the raw projections (q and k above then point at the mapped
    // copies the prep writes, [BH * NC][C][DK] each)
    const u16* qraw;
    const u16* kraw;
    u16* qmap;
    u16* kmap;
    int T, NC, slices, remap, map;
    int H;                // heads (the fixed gate: alpha then holds log gamma [H])
    // the backward's per-chunk records. Forward with REC: st_s the memory entering each chunk
    // [BH * NC][DV][DK], st_u the pseudo-values U and st_r R = V - diag(e^G) K S_in^T
    // [BH * NC][C][DV], all bf16 (o may then be null). Reverse pass: st_s the gradient of the
    // memory leaving each chunk (or null), st_u dU; o receives dV.
    u16* st_s;
    u16* st_u;
    u16* st_r;
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
    static constexpr int TS = C + 8;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    // A is kept as its CT (CT + 1) / 2 lower-triangular 16 x 16 tiles, rows of ATS floats;
    // tile (i, j <= i) at tileA(i, j)
    static constexpr int ATS = 20;
    static constexpr int ATILE = 16 * ATS;
    static constexpr int tileA(int i, int j) { return (i * (i + 1) / 2 + j) * ATILE; }
    // K is dead once A is formed: the diagonal blocks D and T reuse its space
    static constexpr int oK = 0;
    static constexpr int oD = 0;
    static constexpr int oT = oD + al(CT * 256 * 4);
    static constexpr int oA = al(C * KS * 2) > oT + al(C * TS * 2) ? al(C * KS * 2) : oT + al(C * TS * 2);
    static constexpr int oG = oA + al(CT * (CT + 1) / 2 * ATILE * 4);
    static constexpr int oB = oG + al(C * 4);
    static constexpr int bytes = oB + al(C * 4);
    static_assert(bytes <= 64 * 1024, "LDS budget of the delta prep exceeded");
};

template <int C, int DK>
__global__ __launch_bounds__(256, 5)
void delta_tfac_kernel(DspParams p) {
    using Lay = TfacLayout<C, DK>;
    constexpr int CT = C / 16, NT = 256, NW = 4;
    constexpr int KS = Lay::KS, ATS = Lay::ATS, TS = Lay::TS;
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
    // the feature map needs whole rows per aligned lane group (its shuffles need all lanes)
    constexpr bool WHOLE = KP % NT == 0;
    u16x8 rk[KP_PER];
    const u16* kin = p.map ? p.kraw : p.k;
#pragma unroll
    for (int i = 0; i < KP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        const unsigned off = (j < n) ? static_cast<unsigned>(j * DK + col) : 0u;
        rk[i] = *reinterpret_cast<const u16x8*>(kin + tok0 * DK + off);
    }
    if (WHOLE && p.map) {
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
        if (WHOLE || idx < KP) *reinterpret_cast<u16x8*>(sK + j * KS + col) = (j < n) ? rk[i] : z8;
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
        stf4(sA + Lay::tileA(it, jt) + r16 * ATS + 4 * g, a);
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
                const float* arow = sA + Lay::tileA(b, b) + i * ATS;
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
                    const f32x4 a = ldf4(sA + Lay::tileA(i, m) + r16 * ATS + 4 * g);
                    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cvt4(a), cvt4(tcol[m]), acc, 0, 0, 0);
                }
                const f32x4 d = ldf4(sD + i * 256 + r16 * 16 + 4 * g);
                t = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cvt4(-d), cvt4(acc), zf4(), 0, 0, 0);
            }
            tcol[i] = t;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sT[(16 * i + 4 * g + r) * TS + 16 * w + r16] = __builtin_bit_cast(u16, static_cast<__bf16>(t[r] * fu));
            if (p.tfull != nullptr) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.tfull[chunk * C * C + (16 * i + 4 * g + r) * C + 16 * w + r16] =
                        __builtin_bit_cast(u16, static_cast<__bf16>(t[r]));
            }
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
template <int C, int DK, int VS, bool DELTA>
struct DspLayout {
    using TK = SwzTile<DK>;     // K and Q rows
    using TV = SwzTile<VS>;     // the v slice
    static constexpr int NV = VS / 16;
    static constexpr int RS = C + 8;    // T_U and P rows 144 bytes apart: 8-byte row reads of 32 lanes on 64 banks
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    // gate tables of one chunk (floats): G, e^G, e^-G, carry weights e^(G_last - G), then
    // e^(G_last) and G_last
    static constexpr int GG = 0, GEG = C, GENG = 2 * C, GW = 3 * C, GEL = 4 * C, GL = 4 * C + 1;
    static constexpr int KBUF = al(C * TK::STRIDE * 2);
    static constexpr int VBUF = al(C * TV::STRIDE * 2);
    static constexpr int RBUF = al(C * RS * 2);
    static constexpr int GBUF = al((4 * C + 4) * 4);
    // K, Q and the gates of a chunk live three steps (staged, its triangle, its chain), the
    // v slice, T_U (the delta rule only) and the triangle P two
    static constexpr int oK = 0;
    static constexpr int oQ = oK + 3 * KBUF;
    static constexpr int oG = oQ + 3 * KBUF;
    static constexpr int oV = oG + 3 * GBUF;
    static constexpr int oT = oV + 2 * VBUF;
    static constexpr int oP = oT + (DELTA ? 2 * RBUF : 0);
    static constexpr int bytes = oP + 2 * RBUF;
    static_assert(bytes <= 160 * 1024, "LDS budget of the delta single pass exceeded");
};

template <int C, int DK, int DV, int VS, int GK, int VW = 1, bool REV = false, bool REC = false>
__global__ __launch_bounds__(256)
void delta_sp_kernel(DspParams p) {
    constexpr bool DELTA = GK == kGateDeltaRule;
    static_assert(!REV || (DELTA && VW == 1), "the reverse pass is the delta rule's, one value tile per chain wave");
    static_assert(DELTA || GK == kGateScalar || GK == kGateFixed, "scalar gates only");
    static_assert(VW == 1 || (VW == 2 && !DELTA), "two value tiles per chain wave without the delta step only");
    using Lay = DspLayout<C, DK, VS, DELTA>;
    using TK = typename Lay::TK;
    using TV = typename Lay::TV;
    constexpr int NV = Lay::NV;
    constexpr int CT = C / 16, JB = CT / 2;     // token tiles, 32-token blocks
    constexpr int KT = DK / 16, KB = DK / 32;   // key tiles, 32-key blocks
    constexpr int RS = Lay::RS;
    constexpr int NH = 128;                     // helper threads (waves 2 and 3)
    static_assert(C == 64, "the helpers split four token tiles two by two");
    static_assert(DK >= 32 && DK % 32 == 0, "d_k in 32-key blocks");
    static_assert(DV % VS == 0 && (VS == 16 * VW || VS == 32 * VW), "value slices of one or two chain waves");
    // 16-byte pieces of one chunk staged by the helpers: k, q (PKQ each), the v slice (PV),
    // T_U (PT); then one float of G per lane of each helper wave
    constexpr int PKQ = C * DK / 8, PV = C * VS / 8, PT = C * C / 8;
    static_assert(PKQ % NH == 0 && PT % NH == 0 && PV <= 4 * NH, "pieces per helper thread");
    constexpr int NKQ = PKQ / NH, NVP = (PV + NH - 1) / NH, NTP = PT / NH;

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    auto sK = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oK + b * Lay::KBUF); };
    auto sQ = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oQ + b * Lay::KBUF); };
    auto sG = [&](int b) { return reinterpret_cast<float*>(smem + Lay::oG + b * Lay::GBUF); };
    auto sV = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oV + b * Lay::VBUF); };
    auto sT = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oT + b * Lay::RBUF); };
    auto sP = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oP + b * Lay::RBUF); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    // key channels held by a chain wave's memory tile ct at lane group g: chan(ct) + e, e < 4,
    // so that the bf16 operand built from tiles 2b and 2b + 1 holds eight consecutive keys
    // 32b + 8g + 0..7 (one 16-byte LDS read of the matching K or Q row piece)
    auto chan = [&](int ct) { return 32 * (ct >> 1) + 8 * g + 4 * (ct & 1); };
    const int lb = logical_block_of(blockIdx.x, gridDim.x, p.remap);
    const int bh = lb / p.slices, m0 = (lb % p.slices) * VS;
    const int T = p.T, NC = p.NC;
    const int64_t seq0 = static_cast<int64_t>(bh) * T;

    // Global memory through buffer resources, one per tensor and sequence, with the byte offset
    // (lane's part + chunk's part) in the range-checked VGPR offset: reads past the sequence's
    // end return zero and writes past it are dropped, so the tail chunk needs no clamping or
    // masking.
    constexpr int kRsrc = 0x00020000;   // raw buffer, 32-bit data format
    auto rsrc = [](const void* base, int64_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrc);
    };

    if (NC == 0) {
        // T == 0: the memory handed through (every wave of the workgroup leaves here)
        if (w < NV && p.s_out != nullptr) {
            float* so = p.s_out + (static_cast<int64_t>(bh) * DV + m0 + 16 * w + r16) * DK + 4 * g;
            const float* s0 = p.s0 ? p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * w + r16) * DK + 4 * g : nullptr;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) stf4(so + 16 * ct, s0 ? ldf4(s0 + 16 * ct) : zf4());
        }
        return;
    }

    // The per-lane parts of the chains' swizzled K and Q addresses. The tile's swizzle depends
    // on the row mod 16 only, so a row 16 or 32 further down is a constant offset away: every K
    // or Q read of a chunk is one of these (per 32-key block) plus a constant, so the chunk's
    // slot costs one add per block rather than one per read.
    int rowoff[KB > 0 ? KB : 1], troff[KB > 0 ? KB : 1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        rowoff[kb] = TK::off(r16, 32 * kb + 8 * g);                        // rows 16it + r16, keys 32kb + 8g
        troff[kb] = TK::off(4 * g + (r16 >> 2), 32 * kb + 8 * (r16 & 3));   // K^T reads of key block kb
        // (opaque to the compiler: with their low bits known it would join the constants by an
        // or, which no LDS read takes as its offset, and keep one address per read)
        asm volatile("" : "+v"(rowoff[kb]), "+v"(troff[kb]));
    }

    // the triangle of chunk c: P[i][j] = (q_i . k_j) e^(G_i - G_j) for j <= i, zero above, bf16;
    // token tiles IA and IB (compile-time, so the tiles' MFMA chains interleave; IA < 0: tile IB
    // alone), the decays as products of two table entries (FLAT: every G_j of the chunk within
    // 2^+-100) or per element
    auto triangle_tiles = [&](int c, auto ia, auto ib, auto flat) __attribute__((always_inline)) {
        constexpr int IA = decltype(ia)::value, IB = decltype(ib)::value;
        constexpr bool FLAT = decltype(flat)::value;
        constexpr int NJ = IB + 1;   // key row tiles reached (IB > IA)
        constexpr int S0 = IA < 0 ? 1 : 0;   // the first of the two row tiles taken
        const u16* K = sK(c % 3);
        const u16* Q = sQ(c % 3);
        const float* GT = sG(c % 3);
        u16* PP = sP(c & 1);
        bf16x8 qb[2][KB], kr[NJ][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if constexpr (IA >= 0) qb[0][kb] = *reinterpret_cast<const bf16x8*>(Q + TK::off(16 * IA + r16, rr_col(kb, g, KB)));
            qb[1][kb] = *reinterpret_cast<const bf16x8*>(Q + TK::off(16 * IB + r16, rr_col(kb, g, KB)));
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
                kr[jt][kb] = *reinterpret_cast<const bf16x8*>(K + TK::off(16 * jt + r16, rr_col(kb, g, KB)));
        }
        f32x4 dj[NJ], gj[NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) {
            if constexpr (FLAT) dj[jt] = ldf4(GT + Lay::GENG + 16 * jt + 4 * g);
            else gj[jt] = ldf4(GT + Lay::GG + 16 * jt + 4 * g);
        }
        float fi[2];
#pragma unroll
        for (int s = S0; s < 2; ++s) fi[s] = GT[(FLAT ? Lay::GEG : Lay::GG) + 16 * (s == 0 ? IA : IB) + r16];
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc[2][NJ];
#pragma unroll
        for (int s = S0; s < 2; ++s)
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) acc[s][jt] = zf4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int s = S0; s < 2; ++s)
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt)
                    if (jt <= (s == 0 ? IA : IB)) acc[s][jt] = mfma_16x16x32(kr[jt][kb], qb[s][kb], acc[s][jt]);
        // acc[s][jt][e] = q_i . k_j, i = 16 it_s + r16, j = 16jt + 4g + e
#pragma unroll
        for (int s = S0; s < 2; ++s) {
            const int it = s == 0 ? IA : IB;
            const int i = 16 * it + r16;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt) {
                if (jt > it) continue;
                f32x4 d;
                if constexpr (FLAT) {
                    d = dj[jt] * fi[s];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) d[e] = ex2(fi[s] - gj[jt][e]);
                }
                if (jt == it) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * g + e > r16) d[e] = 0.f;
                }
                st4(PP + i * RS + 16 * jt + 4 * g, cvt4(acc[s][jt] * d));
            }
        }
    };
    // With one live chain wave (16-channel slices) chain wave 1 takes token tiles 0 and 1 of
    // the triangle (three 16 x 16 tiles) and the helpers tiles 3 and 2 (four and three): the
    // helpers' step, which bounds the chunk there, gets shorter
    constexpr bool SPLIT3 = !REV && NV <= VW;
    auto triangle01 = [&](int c) __attribute__((always_inline)) {
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        if (sG(c % 3)[Lay::GL] >= -100.f)
            triangle_tiles(c, I0{}, I1{}, std::true_type{});
        else
            triangle_tiles(c, I0{}, I1{}, std::false_type{});
    };

    if (REV && w < 2) {
        // ================================================ reverse pass (the backward)
        // wave w carries the transposed gradient of the memory for value tile w (every key),
        // dacc[ct][e] = dS[m0 + 16w + r16][chan(ct) + e], from the gradient of the final memory
        // back through the chunks (the helpers stage them last first). Per chunk, with dS' the
        // gradient of the memory leaving it (reverse mode through the chain's products):
        //   dU    = P^T dO + diag(e^(G_last - G)) K dS'^T
        //   dR    = T_U^T dU                    (the gradient of V)
        //   dS_in = e^(G_last) dS' + Q^T diag(e^G) dO - K^T diag(e^G) dR    (as dS^T)
        // dS' (bf16 rows) and dU ([C][DV], bf16) go to the workspace for the gradient pass.
        const bool live = w < NV;
        f32x4 dacc[KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            dacc[ct] = zf4();
            if (live && p.s0 != nullptr)
                dacc[ct] = ldf4(p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * w + r16) * DK + chan(ct));
        }
        const auto rdv = rsrc(p.o + seq0 * DV, static_cast<int64_t>(T) * DV * 2);
        const int vrow = m0 + 16 * w + r16;
        lds_barrier();   // the prologue's two barriers
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (live) {
                const int rc = NC - 1 - c;
                const int64_t gc = static_cast<int64_t>(bh) * NC + rc;
                const u16* K = sK(c % 3);
                const u16* Q = sQ(c % 3);
                const float* GT = sG(c % 3);
                const u16* DO = sV(c & 1);
                const u16* TT = sT(c & 1);
                const u16* PP = sP(c & 1);
                bf16x8 ka[CT][KB], pt[CT][JB], tut[CT][JB], qt[KT][JB], kt[KT][JB];
                bf16x4 vv[CT];
                // byte offsets of the K^T and Q^T reads of each key block in this chunk's slot
                // (opaque: each read is one of them plus the instruction's constant offset)
                int ktb[KB > 0 ? KB : 1], qtb[KB > 0 ? KB : 1];
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    ktb[b] = static_cast<int>(reinterpret_cast<const unsigned char*>(K) - smem) + 2 * troff[b];
                    qtb[b] = static_cast<int>(reinterpret_cast<const unsigned char*>(Q) - smem) + 2 * troff[b];
                    asm volatile("" : "+v"(ktb[b]), "+v"(qtb[b]));
                }
                f32x4 eg[CT], wt[CT];
#pragma unroll
                for (int it = 0; it < CT; ++it) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        ka[it][kb] = *reinterpret_cast<const bf16x8*>(K + rowoff[kb] + 16 * it * TK::STRIDE);
                    vv[it] = tr_op_s<VS>(DO, 16 * it, 16 * w, r16, g);   // dO[16it + 4g + e][value r16]
                    eg[it] = ldf4(GT + Lay::GEG + 16 * it + 4 * g);
                    wt[it] = ldf4(GT + Lay::GW + 16 * it + 4 * g);
#pragma unroll
                    for (int b = 0; b < JB; ++b) {
                        // P^T (rows: token j of tile it; slots: tokens i of block b; P's tile
                        // (i-tile, it) exists for i-tile >= it) and T_U^T (rows: token i of tile
                        // it; slots: tokens j of block b; T_U is staged whole, zero above its
                        // diagonal): both by transposed reads of the row-major tiles
                        if (2 * b + 1 < it) continue;
                        pt[it][b] = join8(2 * b >= it ? tr_op<RS>(PP, 32 * b, 16 * it, r16, g) : zero4(),
                                          tr_op<RS>(PP, 32 * b + 16, 16 * it, r16, g));
                        tut[it][b] = join8(tr_op<RS>(TT, 32 * b, 16 * it, r16, g), tr_op<RS>(TT, 32 * b + 16, 16 * it, r16, g));
                    }
                }
#pragma unroll
                for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
                        const int o0 = 2 * (32 * jb * TK::STRIDE + 4 * (ct & 1));
                        kt[ct][jb] = join8(tr4(reinterpret_cast<const u16*>(smem + ktb[ct >> 1] + o0)),
                                           tr4(reinterpret_cast<const u16*>(smem + ktb[ct >> 1] + o0 + 32 * TK::STRIDE)));
                        qt[ct][jb] = join8(tr4(reinterpret_cast<const u16*>(smem + qtb[ct >> 1] + o0)),
                                           tr4(reinterpret_cast<const u16*>(smem + qtb[ct >> 1] + o0 + 32 * TK::STRIDE)));
                    }
                const float dec = GT[Lay::GEL];
                __builtin_amdgcn_sched_barrier(0);

                bf16x8 sb[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sb[kb] = join8(cvt4(dacc[2 * kb]), cvt4(dacc[2 * kb + 1]));
                if (p.st_s != nullptr) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        *reinterpret_cast<bf16x8*>(p.st_s + (gc * DV + vrow) * DK + 32 * kb + 8 * g) = sb[kb];
                }
                // dU[16it + 4g + e][value r16]
                f32x4 du[CT];
#pragma unroll
                for (int it = 0; it < CT; ++it) du[it] = zf4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int it = 0; it < CT; ++it) du[it] = mfma_16x16x32(ka[it][kb], sb[kb], du[it]);
#pragma unroll
                for (int it = 0; it < CT; ++it) {
                    du[it] = du[it] * wt[it];
#pragma unroll
                    for (int b = 0; b < JB; ++b)
                        if (2 * b + 1 >= it) du[it] = mfma_16x16x32(pt[it][b], join8(vv[2 * b], vv[2 * b + 1]), du[it]);
                }
                bf16x8 dub[JB];
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) dub[jb] = join8(cvt4(du[2 * jb]), cvt4(du[2 * jb + 1]));
#pragma unroll
                for (int it = 0; it < CT; ++it) {
                    // (the element bits from the whole vector: a bit cast of one element of a bf16
                    // vector read element 0)
                    const u16x4 b4 = __builtin_bit_cast(u16x4, cvt4(du[it]));
#pragma unroll
                    for (int e = 0; e < 4; ++e) p.st_u[(gc * C + 16 * it + 4 * g + e) * DV + vrow] = b4[e];
                }
                // dR[16it + 4g + e][value r16] (the gradient of v, stored as it stands)
                f32x4 dr[CT];
#pragma unroll
                for (int it = 0; it < CT; ++it) {
                    dr[it] = zf4();
#pragma unroll
                    for (int b = 0; b < JB; ++b)
                        if (2 * b + 1 >= it) dr[it] = mfma_16x16x32(tut[it][b], dub[b], dr[it]);
                    const u16x4 b4 = __builtin_bit_cast(u16x4, cvt4(dr[it]));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __builtin_amdgcn_raw_buffer_store_b16(b4[e], rdv,
                                                              ((rc * C + 16 * it + 4 * g + e) * DV + vrow) * 2, 0, 0);
                }
                // dS^T <- e^(G_last) dS^T + Q^T diag(e^G) dO - K^T diag(e^G) dR
                bf16x8 ob[JB], rn[JB];
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    ob[jb] = join8(cvt4(up4(vv[2 * jb]) * eg[2 * jb]), cvt4(up4(vv[2 * jb + 1]) * eg[2 * jb + 1]));
                    rn[jb] = join8(cvt4(dr[2 * jb] * (-eg[2 * jb])), cvt4(dr[2 * jb + 1] * (-eg[2 * jb + 1])));
                }
#pragma unroll
                for (int ct = 0; ct < KT; ++ct) {
                    f32x4 a = dacc[ct] * dec;
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
                        a = mfma_16x16x32(qt[ct][jb], ob[jb], a);
                        a = mfma_16x16x32(kt[ct][jb], rn[jb], a);
                    }
                    dacc[ct] = a;
                }
            }
            lds_barrier();
        }
        if (live && p.s_out != nullptr) {
#pragma unroll
            for (int ct = 0; ct < KT; ++ct)
                stf4(p.s_out + (static_cast<int64_t>(bh) * DV + vrow) * DK + chan(ct), dacc[ct]);
        }
        return;
    }

    if (w < 2) {
        // ================================================ chain waves
        // wave w < NV / VW carries S^T of value tiles vt = VW w .. VW w + VW - 1 (every key) in
        // fp32 accumulators, sacc[v][ct][e] = S[m0 + 16 vt + r16][chan(ct) + e], and finishes
        // each chunk's outputs for those channels; every product takes the previous one's
        // accumulators as its operand (reduction slots 32b + 4g + e and 32b + 16 + 4g + e).
        // With two tiles per wave the LDS operands (K, Q, P) serve both.
        const bool live = w * VW < NV;
        f32x4 sacc[VW][KT];
#pragma unroll
        for (int v = 0; v < VW; ++v)
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                sacc[v][ct] = zf4();
                if (live && p.s0 != nullptr)
                    sacc[v][ct] = ldf4(p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * (VW * w + v) + r16) * DK + chan(ct));
            }
        const auto ro = rsrc(p.o != nullptr ? p.o + seq0 * DV : nullptr, p.o != nullptr ? static_cast<int64_t>(T) * DV * 2 : 0);
        lds_barrier();   // the prologue's two barriers (between them, the triangle of chunk 0)
        if constexpr (SPLIT3) {
            if (w == 1) triangle01(0);
        }
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (SPLIT3 && !live) {
                if (c + 1 < NC) triangle01(c + 1);   // beside the helpers' part of it
            } else if (live) {
                const u16* K = sK(c % 3);
                const u16* Q = sQ(c % 3);
                const float* GT = sG(c % 3);
                const u16* V = sV(c & 1);
                const u16* TT = sT(c & 1);
                const u16* PP = sP(c & 1);
                // every LDS operand of the chunk is requested before the first product: with one
                // wave per SIMD nothing else hides the LDS latency
                bf16x8 ka[CT][KB], qa[CT][KB], tu[CT][JB], pb[CT][JB], kt[KT][JB];
                bf16x4 vv[VW][CT];
                // byte offsets of the K^T reads of each key block in this chunk's slot, opaque so
                // that each read is one of them plus the instruction's constant offset
                int ktb[KB > 0 ? KB : 1];
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    ktb[b] = static_cast<int>(reinterpret_cast<const unsigned char*>(K) - smem) + 2 * troff[b];
                    asm volatile("" : "+v"(ktb[b]));
                }
                f32x4 eg[CT], wt[CT];
                float egi[CT];
#pragma unroll
                for (int it = 0; it < CT; ++it) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        if constexpr (DELTA) ka[it][kb] = *reinterpret_cast<const bf16x8*>(K + rowoff[kb] + 16 * it * TK::STRIDE);
                        qa[it][kb] = *reinterpret_cast<const bf16x8*>(Q + rowoff[kb] + 16 * it * TK::STRIDE);
                    }
                }
#pragma unroll
                for (int it = 0; it < CT; ++it) {
#pragma unroll
                    for (int v = 0; v < VW; ++v) vv[v][it] = tr_op_s<VS>(V, 16 * it, 16 * (VW * w + v), r16, g);
                    if constexpr (DELTA) eg[it] = ldf4(GT + Lay::GEG + 16 * it + 4 * g);
                    wt[it] = ldf4(GT + Lay::GW + 16 * it + 4 * g);
                    egi[it] = GT[Lay::GEG + 16 * it + r16];
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
                        if (2 * jb > it) continue;
                        const bool hi = 2 * jb + 1 <= it;
                        const u16* tr = TT + (16 * it + r16) * RS + 32 * jb + 4 * g;
                        const u16* pr = PP + (16 * it + r16) * RS + 32 * jb + 4 * g;
                        if constexpr (DELTA) tu[it][jb] = join8(ld4(tr), hi ? ld4(tr + 16) : zero4());
                        pb[it][jb] = join8(ld4(pr), hi ? ld4(pr + 16) : zero4());
                    }
                }
#pragma unroll
                for (int ct = 0; ct < KT; ++ct)
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
                        // A = K^T, row r16 = key 32(ct / 2) + 8(r16 / 4) + 4(ct % 2) + r16 % 4 (the
                        // keys chan(ct) + e of the product's output rows 4g + e), reduction slots
                        // = tokens 32jb + 4g + e and 32jb + 16 + 4g + e: lane (r16, g) reads the
                        // four keys from col of token row 32jb (+16) + 4g + r16 / 4
                        const int o0 = 2 * (32 * jb * TK::STRIDE + 4 * (ct & 1));
                        kt[ct][jb] = join8(tr4(reinterpret_cast<const u16*>(smem + ktb[ct >> 1] + o0)),
                                           tr4(reinterpret_cast<const u16*>(smem + ktb[ct >> 1] + o0 + 32 * TK::STRIDE)));
                    }
                const float dec = GT[Lay::GEL];
                __builtin_amdgcn_sched_barrier(0);

#pragma unroll
                for (int v = 0; v < VW; ++v) {
                    bf16x8 sb[KB];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) sb[kb] = join8(cvt4(sacc[v][2 * kb]), cvt4(sacc[v][2 * kb + 1]));
                    // Y = K S_in^T (y[it][e] = Y[16it + 4g + e][value r16]; the delta rule only)
                    // and o^T = S_in Q^T (oq[it][e] = (S_in q_i)[value 4g + e], i = 16it + r16),
                    // interleaved
                    f32x4 y[CT], oq[CT];
#pragma unroll
                    for (int it = 0; it < CT; ++it) {
                        y[it] = zf4();
                        oq[it] = zf4();
                    }
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int it = 0; it < CT; ++it) {
                            if constexpr (DELTA) y[it] = mfma_16x16x32(ka[it][kb], sb[kb], y[it]);
                            oq[it] = mfma_16x16x32(sb[kb], qa[it][kb], oq[it]);
                        }
                    // the values written: the delta rule's pseudo-values U (R = V - diag(e^G) Y,
                    // then U = T_U R, lower triangular: block jb reaches token tile it when
                    // 2jb <= it) as a bf16 hi + lo pair, else V itself (exact in bf16); weighted
                    // by e^(G_last - G) for the carry
                    bf16x8 uh[JB], ul[JB], wb[JB];
                    if constexpr (DELTA) {
                        bf16x4 rb[CT];
#pragma unroll
                        for (int jt = 0; jt < CT; ++jt) rb[jt] = cvt4(up4(vv[v][jt]) - eg[jt] * y[jt]);
                        f32x4 u[CT];
#pragma unroll
                        for (int it = 0; it < CT; ++it) u[it] = zf4();
#pragma unroll
                        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                            for (int it = 0; it < CT; ++it)
                                if (2 * jb <= it) u[it] = mfma_16x16x32(tu[it][jb], join8(rb[2 * jb], rb[2 * jb + 1]), u[it]);
#pragma unroll
                        for (int jb = 0; jb < JB; ++jb) {
                            const bf16x4 h0 = cvt4(u[2 * jb]), h1 = cvt4(u[2 * jb + 1]);
                            uh[jb] = join8(h0, h1);
                            ul[jb] = join8(cvt4(u[2 * jb] - up4(h0)), cvt4(u[2 * jb + 1] - up4(h1)));
                            wb[jb] = join8(cvt4(u[2 * jb] * wt[2 * jb]), cvt4(u[2 * jb + 1] * wt[2 * jb + 1]));
                        }
                        if constexpr (REC) {
                            // the backward's records of the chunk: S_in rows (keys 32kb + 8g .. + 7
                            // of value row vrow), U and R at (token 16it + 4g + e, value vrow)
                            const int64_t gc = static_cast<int64_t>(bh) * NC + c;
                            const int vrow = m0 + 16 * (VW * w + v) + r16;
#pragma unroll
                            for (int kb = 0; kb < KB; ++kb)
                                *reinterpret_cast<bf16x8*>(p.st_s + (gc * DV + vrow) * DK + 32 * kb + 8 * g) = sb[kb];
#pragma unroll
                            for (int it = 0; it < CT; ++it) {
                                // (element bits from the whole vector: a bit cast of one element of a
                                // bf16 vector read element 0)
                                const u16x4 ub = __builtin_bit_cast(u16x4, cvt4(u[it])), rr = __builtin_bit_cast(u16x4, rb[it]);
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int64_t at = (gc * C + 16 * it + 4 * g + e) * DV + vrow;
                                    p.st_u[at] = ub[e];
                                    p.st_r[at] = rr[e];
                                }
                            }
                        }
                    } else {
#pragma unroll
                        for (int jb = 0; jb < JB; ++jb) {
                            uh[jb] = join8(vv[v][2 * jb], vv[v][2 * jb + 1]);
                            wb[jb] = join8(cvt4(up4(vv[v][2 * jb]) * wt[2 * jb]), cvt4(up4(vv[v][2 * jb + 1]) * wt[2 * jb + 1]));
                        }
                    }
                    // carry S^T <- e^(G_last) S^T + K^T diag(e^(G_last - G)) U and outputs
                    // o^T = S_in Q^T diag(e^G) + U^T P^T, interleaved
                    f32x4 ot[CT];
#pragma unroll
                    for (int it = 0; it < CT; ++it) ot[it] = oq[it] * egi[it];
#pragma unroll
                    for (int ct = 0; ct < KT; ++ct) sacc[v][ct] = sacc[v][ct] * dec;
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
                        for (int ct = 0; ct < KT; ++ct) sacc[v][ct] = mfma_16x16x32(kt[ct][jb], wb[jb], sacc[v][ct]);
#pragma unroll
                        for (int it = 0; it < CT; ++it) {
                            if (2 * jb > it) continue;
                            ot[it] = mfma_16x16x32(uh[jb], pb[it][jb], ot[it]);
                            if constexpr (DELTA) ot[it] = mfma_16x16x32(ul[jb], pb[it][jb], ot[it]);
                        }
                    }
                    // o[16it + r16][m0 + 16vt + 4g + e]
                    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
                    for (int it = 0; it < CT; ++it)
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, cvt4(ot[it])), ro,
                                                              ((c * C + 16 * it + r16) * DV + m0 + 16 * (VW * w + v) + 4 * g) * 2,
                                                              0, 0);
                }
            }
            lds_barrier();
        }
        if (live && p.s_out != nullptr) {
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                float* so = p.s_out + (static_cast<int64_t>(bh) * DV + m0 + 16 * (VW * w + v) + r16) * DK;
#pragma unroll
                for (int ct = 0; ct < KT; ++ct) stf4(so + chan(ct), sacc[v][ct]);
            }
        }
        return;
    }

    // ================================================ helper waves
    // every global load of the pass (the same ones in both waves, so the compiler's count of
    // loads in flight is exact), the staging of each chunk, and the decayed triangle P one
    // chunk ahead of the chain: wave 2 token tiles {0, 3}, wave 3 {1, 2} (five tiles each)
    const int ht = tid - 128;                      // 0 .. 127
    const int hw = w - 2;
    const auto rk = rsrc(p.k + static_cast<int64_t>(bh) * p.qk_seq * DK, static_cast<int64_t>(p.qk_seq) * DK * 2);
    const auto rq = rsrc(p.q + static_cast<int64_t>(bh) * p.qk_seq * DK, static_cast<int64_t>(p.qk_seq) * DK * 2);
    const auto rv = rsrc(p.v + seq0 * DV, static_cast<int64_t>(T) * DV * 2);
    const int64_t chunk0 = static_cast<int64_t>(bh) * NC;
    // the delta rule's T_U and cumulative gates from its prep; the scalar gate's raw log
    // alpha (zero past the sequence's end, so that the cumulative sums stay flat there)
    const auto rt = rsrc(DELTA ? p.tu + chunk0 * C * C : nullptr, DELTA ? static_cast<int64_t>(NC) * C * C * 2 : 0);
    const auto rgt = DELTA ? rsrc(p.g + chunk0 * C, static_cast<int64_t>(NC) * C * 4)
                           : rsrc(GK == kGateScalar ? p.alpha + seq0 : nullptr, GK == kGateScalar ? static_cast<int64_t>(T) * 4 : 0);
    const float lg2 = GK == kGateFixed ? p.alpha[bh % p.H] * kLog2e : 0.f;   // log2 of the fixed decay

    // the register ring: K, Q and G of chunk a, the v slice and T_U of chunk b
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    struct Entry {
        u32x4 k[NKQ], q[NKQ], v[NVP], t[NTP];
        float g;
    };
    Entry ring[2];
    auto load = [&](Entry& e, int a, int b) {
        if constexpr (REV) {
            // the reverse pass stages the chunks last first
            a = NC - 1 - a;
            b = NC - 1 - b;
        }
#pragma unroll
        for (int i = 0; i < NKQ; ++i) {
            const int pc = ht + i * NH, j = pc / (DK / 8), col = (pc % (DK / 8)) * 8;
            e.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, ((a * C + j) * DK + col) * 2, 0, 0);
            e.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, ((a * C + j) * DK + col) * 2, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NVP; ++i) {
            const int pc = (ht + i * NH) % PV, j = pc / (VS / 8), col = (pc % (VS / 8)) * 8;
            e.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((b * C + j) * DV + m0 + col) * 2, 0, 0);
        }
        if constexpr (DELTA) {
#pragma unroll
            for (int i = 0; i < NTP; ++i)
                e.t[i] = __builtin_amdgcn_raw_buffer_load_b128(rt, b * C * C * 2 + (ht + i * NH) * 16, 0, 0);
        }
        if constexpr (GK != kGateFixed)
            e.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgt, (a * C + lane) * 4, 0, 0));
    };
    // K, Q, G of chunk a into slot set sa (mod 3); the v slice and T_U into slot set sb (mod 2)
    auto stage_kqg = [&](const Entry& e, int sa) {
        u16* K = sK(sa % 3);
        u16* Q = sQ(sa % 3);
#pragma unroll
        for (int i = 0; i < NKQ; ++i) {
            const int pc = ht + i * NH, j = pc / (DK / 8), col = (pc % (DK / 8)) * 8;
            *reinterpret_cast<u32x4*>(K + TK::off(j, col)) = e.k[i];
            *reinterpret_cast<u32x4*>(Q + TK::off(j, col)) = e.q[i];
        }
        if (hw == 0) {
            // gate tables: lane t holds G_t (log2 units, flat past the end of the sequence):
            // the delta rule's from its prep, the scalar gate's scanned here, the fixed gate's
            // (min(t, n - 1) + 1) log2 gamma
            float* GT = sG(sa % 3);
            float G;
            if constexpr (DELTA) {
                G = e.g;
            } else if constexpr (GK == kGateScalar) {
                G = wave_inclusive_scan_dpp(e.g * kLog2e);
            } else {
                const int n = T - sa * C;
                G = static_cast<float>((lane < n ? lane : (n > 0 ? n - 1 : 0)) + 1) * lg2;
            }
            const float gl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), C - 1));
            GT[Lay::GG + lane] = G;
            GT[Lay::GEG + lane] = ex2(G);
            GT[Lay::GENG + lane] = ex2(-G);
            GT[Lay::GW + lane] = ex2(gl - G);
            if (lane == 0) {
                GT[Lay::GEL] = ex2(gl);
                GT[Lay::GL] = gl;
            }
        }
    };
    auto stage_vt = [&](const Entry& e, int sb) {
        u16* V = sV(sb & 1);
        u16* TT = sT(sb & 1);
#pragma unroll
        for (int i = 0; i < NVP; ++i) {
            const int pc = ht + i * NH;
            if (PV % NH == 0 || pc < PV) {
                const int j = pc / (VS / 8), col = (pc % (VS / 8)) * 8;
                *reinterpret_cast<u32x4*>(V + TV::off(j, col)) = e.v[i];
            }
        }
        if constexpr (DELTA) {
#pragma unroll
            for (int i = 0; i < NTP; ++i) {
                const int pc = ht + i * NH, row = pc / (C / 8), col = (pc % (C / 8)) * 8;
                *reinterpret_cast<u32x4*>(TT + row * RS + col) = e.t[i];
            }
        }
    };
    auto triangle = [&](int c) __attribute__((always_inline)) {
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using IN = std::integral_constant<int, -1>;
        const bool flat = sG(c % 3)[Lay::GL] >= -100.f;
        if constexpr (SPLIT3) {
            if (hw == 0) {
                if (flat) triangle_tiles(c, IN{}, I3{}, std::true_type{});
                else triangle_tiles(c, IN{}, I3{}, std::false_type{});
            } else {
                if (flat) triangle_tiles(c, IN{}, I2{}, std::true_type{});
                else triangle_tiles(c, IN{}, I2{}, std::false_type{});
            }
        } else if (hw == 0) {
            if (flat) triangle_tiles(c, I0{}, I3{}, std::true_type{});
            else triangle_tiles(c, I0{}, I3{}, std::false_type{});
        } else {
            if (flat) triangle_tiles(c, I1{}, I2{}, std::true_type{});
            else triangle_tiles(c, I1{}, I2{}, std::false_type{});
        }
    };

    // prologue: K, Q, G of chunks 0 and 1, the v slice and T_U of chunk 0, the triangle of chunk 0
    const int last = NC - 1;
    load(ring[0], 0, 0);
    load(ring[1], last > 0 ? 1 : 0, 0);
    stage_kqg(ring[0], 0);
    stage_vt(ring[0], 0);
    stage_kqg(ring[1], 1);
    lds_barrier();
    triangle(0);
    load(ring[1], last > 1 ? 2 : last, last > 0 ? 1 : 0);
    lds_barrier();
    // step c (ring slot R = c & 1): loads of K, Q, G of chunk c + 3 and the v slice and T_U of
    // chunk c + 2; the triangle of chunk c + 1; staging of the other slot (K, Q, G of chunk
    // c + 2 into slot set c + 2, the v slice and T_U of chunk c + 1 into slot set c + 1). Past
    // the end the chunks are clamped to the last one and staged into slots no wave reads again.
    auto step = [&](int c, auto slot) __attribute__((always_inline)) {
        constexpr int R = decltype(slot)::value;
        load(ring[R], c + 3 < NC ? c + 3 : last, c + 2 < NC ? c + 2 : last);
        if (c + 1 < NC) triangle(c + 1);
        stage_kqg(ring[R ^ 1], c + 2);
        stage_vt(ring[R ^ 1], c + 1);
        lds_barrier();
    };
    int c = 0;
    for (; c + 1 < NC; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        step(c + 1, std::integral_constant<int, 1>{});
    }
    if (c < NC) step(c, std::integral_constant<int, 0>{});
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

// Layer norm of bf16 output rows in place (the output norm of retention and the scalar decay
// when fused in): the row's mean, then its variance about the mean, both over the DV values
// in fp32; o <- (o - mean) / sqrt(var + eps) * weight + bias (bias may be null). Lanes as in
// rms_rows_bf16_kernel.
template <int DV>
__global__ __launch_bounds__(256)
void layernorm_rows_bf16_kernel(u16* o, const float* weight, const float* bias, float eps, int64_t rows) {
    constexpr int PER = DV / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t row = (static_cast<int64_t>(blockIdx.x) * 256 + tid) / 16;
    const int part = lane & 15;
    const bool live = row < rows;
    u16* r = o + (live ? row : 0) * DV + part * PER;
    float x[PER];
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        x[e] = bf16_bits_to_f32(r[e]);
        s += x[e];
    }
    const float mean = row16_sum(s) / static_cast<float>(DV);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) ss += (x[e] - mean) * (x[e] - mean);
    const float inv = 1.f / __builtin_sqrtf(row16_sum(ss) / static_cast<float>(DV) + eps);
    // the scale and shift of this lane's channels, loaded outside the store loop (a load under
    // a condition there keeps the row's stores from merging into one)
    float wv[PER], bv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        wv[e] = weight[part * PER + e];
        bv[e] = 0.f;
    }
    if (bias != nullptr) {
#pragma unroll
        for (int e = 0; e < PER; ++e) bv[e] = bias[part * PER + e];
    }
    if (live) {
#pragma unroll
        for (int e = 0; e < PER; ++e) r[e] = f32_to_bf16_bits((x[e] - mean) * inv * wv[e] + bv[e]);
    }
}

// The output norm as a pass over bf16 rows [rows][DV]: RMS (fuse bit 1) or layer norm (bit 2).
template <int DV>
hipError_t launch_norm_rows_bf16(const ChunkArgs& a, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(a.B) * a.H * a.T;
    if (rows == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((rows * 16 + 255) / 256));
    if (a.fuse & 4)
        hipLaunchKernelGGL((layernorm_rows_bf16_kernel<DV>), grid, dim3(256), 0, stream, static_cast<u16*>(a.o), a.onw,
                           a.onb, a.oeps, rows);
    else
        hipLaunchKernelGGL((rms_rows_bf16_kernel<DV>), grid, dim3(256), 0, stream, static_cast<u16*>(a.o), a.onw, a.oeps,
                           rows);
    return hipGetLastError();
}

// ====================================================================== launch
template <int C, int DK, int DV>
hipError_t launch_dsp_dv(const ChunkArgs& a, hipStream_t stream) {
    constexpr int VS = DV >= 32 ? 32 : 16;
    const int NC = (a.T + C - 1) / C;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    DspParams p{};
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
    hipLaunchKernelGGL((delta_sp_kernel<C, DK, DV, VS, kGateDeltaRule>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
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

// Retention (GK = kGateFixed) and the scalar decay (kGateScalar) on the same single pass: no
// prep (the helpers form the gate tables from log gamma or the raw log alpha), U = V. Slices
// of 64 value channels (two chain waves of two value tiles) when that still gives every CU a
// workgroup, else 32 (two chain waves of one), else 16.
template <int C, int DK, int DV, int GK, int VS, int VW>
hipError_t launch_lsp_vs(const ChunkArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    DspParams p{};
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.alpha = a.gate;
    p.s0 = a.s0;
    p.o = static_cast<u16*>(a.o);
    p.s_out = a.s_out;
    p.T = a.T;
    p.NC = (a.T + C - 1) / C;
    p.H = a.H;
    p.qk_seq = a.T;
    p.slices = DV / VS;
    const int64_t grid = heads * p.slices;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((delta_sp_kernel<C, DK, DV, VS, GK, VW>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int C, int DK, int DV, int GK>
hipError_t launch_lsp_dv(const ChunkArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if constexpr (DV >= 64) {
        if (heads * (DV / 64) >= kCUs) return launch_lsp_vs<C, DK, DV, GK, 64, 2>(a, stream);
    }
    if constexpr (DV >= 32) {
        if (heads * (DV / 32) >= kCUs) return launch_lsp_vs<C, DK, DV, GK, 32, 1>(a, stream);
    }
    return launch_lsp_vs<C, DK, DV, GK, 16, 1>(a, stream);
}

template <int C, int GK>
hipError_t launch_lsp(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk * 1000 + a.dv) {
        case 32016: return launch_lsp_dv<C, 32, 16, GK>(a, stream);
        case 32032: return launch_lsp_dv<C, 32, 32, GK>(a, stream);
        case 32064: return launch_lsp_dv<C, 32, 64, GK>(a, stream);
        case 32128: return launch_lsp_dv<C, 32, 128, GK>(a, stream);
        case 64016: return launch_lsp_dv<C, 64, 16, GK>(a, stream);
        case 64032: return launch_lsp_dv<C, 64, 32, GK>(a, stream);
        case 64064: return launch_lsp_dv<C, 64, 64, GK>(a, stream);
        case 64128: return launch_lsp_dv<C, 64, 128, GK>(a, stream);
        case 128016: return launch_lsp_dv<C, 128, 16, GK>(a, stream);
        case 128032: return launch_lsp_dv<C, 128, 32, GK>(a, stream);
        case 128064: return launch_lsp_dv<C, 128, 64, GK>(a, stream);
        case 128128: return launch_lsp_dv<C, 128, 128, GK>(a, stream);
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
