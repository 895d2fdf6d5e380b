// Gated delta rule, chunked forward with bf16 storage: three kernels.
//
// Method: the gated delta rule ("Scrivere meglio nella memoria", section
// "Unire oblio e correzione: Gated DeltaNet") in the chunkwise form of the
// RetNet page (section "RetNet: la retention e le sue tre forme", Fig. 16.5),
// with the pseudo-values of the WY / UT representation (section "Correggere:
// la delta rule": one triangular system per chunk, only the end-of-chunk memory
// passed on). Per chunk of n tokens, local inclusive cumulative log-gates G,
// Gamma_ij = e^(G_i - G_j):
//   A   = strictly_lower(diag(beta) (K K^T . Gamma)),  T = (I + A)^-1
//   W   = T diag(beta e^G) K,   U0 = T diag(beta) V
//   U   = U0 - W S_in^T
//   o_i = e^(G_i) S_in q_i + sum_{j<=i} Gamma_ij (q_i.k_j) u_j
//   S_out = e^(G_{n-1}) S_in + sum_j e^(G_{n-1} - G_j) u_j k_j^T
// Everything except U and the carry is independent of the memory, so:
//   prep    (all chunks in parallel) G, A, T's diagonal blocks, W and U0 by
//           blocked forward substitution on MFMA; W (bf16, token-major), U0
//           (fp32, value-major) and G go to the workspace;
//   state   (chunks in order) per chunk: store S_in (bf16), U = U0 - W S_in^T with
//           the memory straight from the accumulators as the B operand, then the
//           carry K^T (weighted U);
//   output  (all chunks in parallel) U = U0 - W S_in^T again from the stored bf16
//           memory (the same operands the state pass used), P = (Q K^T . Gamma)
//           masked, o = e^G S_in q + P U, U entering as a bf16 hi + lo pair (its
//           rounding would otherwise dominate the output error).
#pragma once

#include "chunk_common.hpp"

namespace glr {
namespace ck {

// Workspace of one call: per (sequence, chunk) W [C][DK] bf16, U [DV][C] fp32,
// G [C] fp32 and the memory entering the chunk S [DV][DK] bf16, each array
// contiguous over (sequence, chunk); with the fused feature map also the mapped
// keys KN [C][DK] bf16 (written by the prep, read by the other two kernels).
struct DeltaWs {
    u16* w;
    float* u;
    float* g;
    u16* s;
    u16* kn;
};

inline size_t delta_ws_align(size_t x) { return (x + 255) / 256 * 256; }

inline size_t delta_ws_bytes(int64_t chunks, int C, int dk, int dv, bool mapped_keys) {
    return delta_ws_align(chunks * C * dk * 2) + delta_ws_align(chunks * dv * C * 4) + delta_ws_align(chunks * C * 4) +
           delta_ws_align(chunks * dv * dk * 2) + (mapped_keys ? delta_ws_align(chunks * C * dk * 2) : 0);
}

inline DeltaWs delta_ws_split(void* base, int64_t chunks, int C, int dk, int dv) {
    unsigned char* b = static_cast<unsigned char*>(base);
    DeltaWs ws;
    ws.w = reinterpret_cast<u16*>(b);
    b += delta_ws_align(chunks * C * dk * 2);
    ws.u = reinterpret_cast<float*>(b);
    b += delta_ws_align(chunks * dv * C * 4);
    ws.g = reinterpret_cast<float*>(b);
    b += delta_ws_align(chunks * C * 4);
    ws.s = reinterpret_cast<u16*>(b);
    b += delta_ws_align(chunks * dv * dk * 2);
    ws.kn = reinterpret_cast<u16*>(b);   // only inside the workspace with the fused feature map
    return ws;
}

struct DeltaParams {
    const u16* q;         // [BH][T][DK]
    const u16* k;         // [BH][T][DK]
    const u16* v;         // [BH][T][DV]
    const float* alpha;   // log alpha [BH][T]
    const float* beta;    // [BH][T]
    const float* s0;      // [BH][DV][DK] or null
    u16* o;               // [BH][T][DV]
    float* s_out;         // [BH][DV][DK] or null
    DeltaWs ws;
    int T, NC, vblocks;
    int fuse;             // bit 0: SiLU + L2 on q, k; bit 1: RMS norm of o (weight onw, eps oeps)
    const float* onw;     // [DV] or null
    float oeps;
};

// ====================================================================== prep
//
// One workgroup (four waves) per (sequence, chunk). With T = (I + A)^-1 the two
// right-hand sides differ only by a diagonal on the right of T, so the kernel forms
// T itself (block lower triangular) with beta and beta e^G folded into its columns,
//   T_U = T diag(beta),   T_W = T diag(beta e^G),   U0 = T_U V,   W = T_W K,
// and the two products are plain MFMA contractions over the chunk, independent for
// every output tile. Steps (a workgroup barrier between each):
//   stage k, v; cumulative gates (wave prefix scan)
//   A tiles (K K^T . Gamma, row-scaled by beta, strictly lower) in fp32
//   T's diagonal blocks D_b = (I + A_bb)^-1 by forward substitution (one wave)
//   T's off-diagonal blocks, one column block per wave:
//       T_iw = -D_i sum_{w <= m < i} A_im T_mw,   T_ww = D_w
//   U0 tiles (stored value-major, fp32) and W tiles (through LDS, stored
//   token-major, bf16).
template <int C, int DK, int DV>
struct PrepLayout {
    static constexpr int CT = C / 16;
    static constexpr int KS = tile_stride(DK);   // staged k (natural and transposed reads)
    static constexpr int VS = tile_stride(DV);   // staged v (transposed reads)
    static constexpr int WS = DK + 8;            // W staged for coalesced stores
    static constexpr int AS = C + 4;             // A, fp32
    static constexpr int TS = C + 4;             // T_U, T_W, bf16
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int mx(int a, int b) { return a > b ? a : b; }
    static constexpr int oK = 0;
    static constexpr int oV = oK + al(C * KS * 2);
    static constexpr int oA = oV + al(C * VS * 2);     // A, later W (A is dead by then)
    static constexpr int oD = oA + mx(al(C * AS * 4), al(C * WS * 2));
    static constexpr int oTU = oD + al(CT * 256 * 4);
    static constexpr int oTW = oTU + al(C * TS * 2);
    static constexpr int oG = oTW + al(C * TS * 2);
    static constexpr int oB = oG + al(C * 4);
    static constexpr int bytes = oB + al(C * 4);
    static_assert(bytes <= 160 * 1024, "LDS budget of the prep kernel exceeded");
};

template <int C, int DK, int DV>
__global__ __launch_bounds__(256)
void delta_prep_kernel(DeltaParams p) {
    using Lay = PrepLayout<C, DK, DV>;
    constexpr int CT = C / 16, NT = 256, NW = 4;
    constexpr int KS = Lay::KS, VS = Lay::VS, WS = Lay::WS, AS = Lay::AS, TS = Lay::TS;
    constexpr int KB = (DK + 31) / 32;
    constexpr int KP = C * DK / 8, KP_PER = (KP + NT - 1) / NT;
    constexpr int VP = C * DV / 8, VP_PER = (VP + NT - 1) / NT;
    constexpr int NPAIR = CT * (CT + 1) / 2;
    constexpr int NTW = DK / 16, NTU = DV / 16, NTT = NTW + NTU, NT_PER = (NTT + NW - 1) / NW;
    static_assert(CT <= NW, "one wave per column block of T");

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    u16* const sV = reinterpret_cast<u16*>(smem + Lay::oV);
    float* const sA = reinterpret_cast<float*>(smem + Lay::oA);
    u16* const sW = reinterpret_cast<u16*>(smem + Lay::oA);
    float* const sD = reinterpret_cast<float*>(smem + Lay::oD);
    u16* const sTU = reinterpret_cast<u16*>(smem + Lay::oTU);
    u16* const sTW = reinterpret_cast<u16*>(smem + Lay::oTW);
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

    // ---- stage k, v (rows past the end zero); cumulative gates and write strengths
    u16x8 rk[KP_PER], rv[VP_PER];
#pragma unroll
    for (int i = 0; i < KP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        const unsigned off = (idx < KP && j < n) ? static_cast<unsigned>(j * DK + col) : 0u;
        rk[i] = *reinterpret_cast<const u16x8*>(p.k + tok0 * DK + off);
    }
#pragma unroll
    for (int i = 0; i < VP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
        const unsigned off = (idx < VP && j < n) ? static_cast<unsigned>(j * DV + col) : 0u;
        rv[i] = *reinterpret_cast<const u16x8*>(p.v + tok0 * DV + off);
    }
    if (w == 0) {
        float la = 0.f, be = 0.f;
        if (lane < n) {
            la = p.alpha[tok0 + lane] * kLog2e;
            be = p.beta[tok0 + lane];
        }
        const float G = wave_inclusive_scan(la);   // padded tokens carry a zero log-gate
        if (lane < C) {
            sG[lane] = G;
            sBeta[lane] = be;
            p.ws.g[chunk * C + lane] = G;
        }
    }
#pragma unroll
    for (int i = 0; i < KP_PER; ++i) {
        const int idx = tid + i * NT;
        const u16x8 x = (p.fuse & 1) ? silu_l2_piece<DK / 8>(rk[i]) : rk[i];
        if (idx < KP) {
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            *reinterpret_cast<u16x8*>(sK + j * KS + col) = (j < n) ? x : z8;
            // the mapped keys for the state and output passes (rows past the end zero)
            if (p.fuse & 1) *reinterpret_cast<u16x8*>(p.ws.kn + chunk * C * DK + j * DK + col) = (j < n) ? x : z8;
        }
    }
#pragma unroll
    for (int i = 0; i < VP_PER; ++i) {
        const int idx = tid + i * NT;
        if (idx < VP) {
            const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            *reinterpret_cast<u16x8*>(sV + j * VS + col) = (j < n) ? rv[i] : z8;
        }
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

    // ---- T's diagonal 16 x 16 blocks D_b = (I + A_bb)^-1 by forward substitution
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

    // ---- column block w of T: lane (r16, g) holds T[16i + 4g + r][16w + r16];
    // written as T_U and T_W with the column's factor
    if (w < CT) {
        const float fu = sBeta[16 * w + r16];
        const float fw = fu * ex2(sG[16 * w + r16]);
        f32x4 tcol[CT];
#pragma unroll
        for (int i = 0; i < CT; ++i) {
            if (i < w) continue;
            f32x4 t;
            if (i == w) {
#pragma unroll
                for (int r = 0; r < 4; ++r) t[r] = sD[w * 256 + (4 * g + r) * 16 + r16];
            } else {
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
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * g + r;
                sTU[row * TS + 16 * w + r16] = __builtin_bit_cast(u16, static_cast<__bf16>(t[r] * fu));
                sTW[row * TS + 16 * w + r16] = __builtin_bit_cast(u16, static_cast<__bf16>(t[r] * fw));
            }
        }
    }
    lds_barrier();

    // ---- U0 = T_U V (value-major fp32 to the workspace), W = T_W K (through LDS):
    // row block it of T contracts over the 16(it + 1) tokens it reaches
    float* const ug = p.ws.u + chunk * DV * C;
#pragma unroll
    for (int s = 0; s < NT_PER; ++s) {
        const int nt = w + NW * s;
        if (nt >= NTT) break;
        const bool isw = nt < NTW;
        const u16* const tmat = isw ? sTW : sTU;
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            f32x4 acc = zf4();
#pragma unroll
            for (int kb = 0; kb < (CT + 1) / 2; ++kb) {
                if (2 * kb > it) continue;
                const bool hi = 2 * kb + 1 <= it;
                const u16* trow = tmat + (16 * it + r16) * TS + 32 * kb + 4 * g;
                const bf16x8 tb = join8(ld4(trow), hi ? ld4(trow + 16) : zero4());
                if (isw) acc = mfma_16x16x32(tr_split<KS>(sK, kb, 16 * nt, hi, r16, g), tb, acc);
                else acc = mfma_16x16x32(tb, tr_split<VS>(sV, kb, 16 * (nt - NTW), hi, r16, g), acc);
            }
            if (isw) {
                // acc[r] = W[16it + r16][16nt + 4g + r]
                st4(sW + (16 * it + r16) * WS + 16 * nt + 4 * g, cvt4(acc));
            } else {
                // acc[r] = U0[16it + 4g + r][16(nt - NTW) + r16]
                stf4(ug + (16 * (nt - NTW) + r16) * C + 16 * it + 4 * g, acc);
            }
        }
    }
    lds_barrier();
    u16* const wg = p.ws.w + chunk * C * DK;
#pragma unroll
    for (int i = 0; i < KP_PER; ++i) {
        const int idx = tid + i * NT;
        if (idx < KP) {
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            *reinterpret_cast<u16x8*>(wg + j * DK + col) = *reinterpret_cast<const u16x8*>(sW + j * WS + col);
        }
    }
}

// ====================================================================== state
//
// Workgroup: NVT value tiles x NKH key groups of waves. Wave (vt, kh) keeps the
// memory for value tile vt and key tiles kh*KTW .. kh*KTW + KTW - 1 in fp32 MFMA
// accumulators: sacc[t][r] = S[16 vt' + r16][16(kh KTW + t) + 4g + r]. Per chunk
// (two workgroup barriers, W and K double-buffered in LDS):
//   phase 1  store the entering memory (bf16); partial W S^T over the wave's key
//            tiles with the accumulators as the B operand; the key group 0 wave
//            adds U0 (requested a chunk ahead); partials to LDS;
//   phase 2  U = sum of the key groups' partials; the carry
//            S^T <- e^(G_last) S^T + K^T (e^(G_last - G_j) u_j) with K^T read
//            transposed from LDS; the next chunk is staged and the one after
//            requested.
// U itself is not stored: the output pass forms it again from U0, W and the stored
// memory, which costs less HBM traffic than writing and re-reading it.
template <int C, int DK, int NVT, int NKH>
struct DStateLayout {
    static constexpr int WS = DK + 8;                 // W, natural 8-byte reads
    static constexpr int KS = tile_stride(DK);   // K, transposed reads
    static constexpr int XS = C + 4;                  // partials, [value][token] fp32
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int WB = al(C * WS * 2), KB_ = al(C * KS * 2), GB = al(C * 4);
    static constexpr int BUF = WB + KB_ + GB;         // one staged chunk
    static constexpr int oX = 2 * BUF;
    static constexpr int bytes = oX + (NKH > 1 ? al(NVT * NKH * 16 * XS * 4) : 0);
    static_assert(bytes <= 160 * 1024, "LDS budget of the delta state pass exceeded");
};

template <int C, int DK, int DV, int NVT, int NKH>
__global__ __launch_bounds__(64 * NVT * NKH)
void delta_state_kernel(DeltaParams p) {
    using Lay = DStateLayout<C, DK, NVT, NKH>;
    constexpr int NW = NVT * NKH, NT = 64 * NW;
    constexpr int CT = C / 16, JB = (CT + 1) / 2;
    constexpr int KT = DK / 16, KTW = KT / NKH;
    static_assert(KT % NKH == 0 && (KTW % 2 == 0 || KTW == 1), "key tiles per wave: even, or a single one");
    constexpr int WS = Lay::WS, KS = Lay::KS, XS = Lay::XS;
    constexpr int KP = C * DK / 8, KP_PER = (KP + NT - 1) / NT;

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    auto sW = [&](int b) { return reinterpret_cast<u16*>(smem + b * Lay::BUF); };
    auto sK = [&](int b) { return reinterpret_cast<u16*>(smem + b * Lay::BUF + Lay::WB); };
    auto sG = [&](int b) { return reinterpret_cast<float*>(smem + b * Lay::BUF + Lay::WB + Lay::KB_); };
    float* const sX = reinterpret_cast<float*>(smem + Lay::oX);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int vt = wave % NVT, kh = wave / NVT;
    const int r16 = lane & 15, g = lane >> 4;

    // the value blocks of one head run on one XCD and share its L2 copy of W and K
    const int lb = logical_block_of(blockIdx.x, gridDim.x, (gridDim.x & 7) == 0);
    const int bh = lb / p.vblocks;
    const int v0 = (lb % p.vblocks) * 16 * NVT + 16 * vt;   // this wave's value tile
    const int T = p.T, NC = p.NC;
    const int64_t tok0 = static_cast<int64_t>(bh) * T;
    const int key0 = 16 * KTW * kh;

    f32x4 sacc[KTW];
    {
        const float* s0 = p.s0 ? p.s0 + (static_cast<int64_t>(bh) * DV + v0 + r16) * DK + key0 + 4 * g : nullptr;
#pragma unroll
        for (int t = 0; t < KTW; ++t) sacc[t] = s0 ? ldf4(s0 + 16 * t) : zf4();
    }
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    auto chunk_len = [&](int c) { return (T - c * C < C) ? (T - c * C) : C; };

    // the next chunk's W and K pieces and gates in registers (chunk clamped past the end)
    u16x8 rw[KP_PER], rk[KP_PER];
    float rg = 0.f;
    auto fetch = [&](int cr) {
        const int c = cr < NC ? cr : NC - 1;
        const int n = chunk_len(c);
        const u16* wc = p.ws.w + (static_cast<int64_t>(bh) * NC + c) * C * DK;
        const u16* kc = (p.fuse & 1) ? p.ws.kn + (static_cast<int64_t>(bh) * NC + c) * C * DK
                                     : p.k + (tok0 + static_cast<int64_t>(c) * C) * DK;
#pragma unroll
        for (int i = 0; i < KP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const unsigned off = (idx < KP && j < n) ? static_cast<unsigned>(j * DK + col) : 0u;
            rw[i] = *reinterpret_cast<const u16x8*>(wc + off);
            rk[i] = *reinterpret_cast<const u16x8*>(kc + off);
        }
        rg = p.ws.g[(static_cast<int64_t>(bh) * NC + c) * C + (tid < C ? tid : 0)];
    };
    auto stage = [&](int b, int c) {
        const int n = chunk_len(c);
#pragma unroll
        for (int i = 0; i < KP_PER; ++i) {
            const int idx = tid + i * NT;
            if (KP % NT == 0 || idx < KP) {
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                *reinterpret_cast<u16x8*>(sW(b) + j * WS + col) = (j < n) ? rw[i] : z8;
                *reinterpret_cast<u16x8*>(sK(b) + j * KS + col) = (j < n) ? rk[i] : z8;
            }
        }
        if (tid < C) sG(b)[tid] = rg;
    };

    // U0 of the next chunk (key group 0 only), requested a chunk ahead: chunk c's U0 is
    // consumed right after its W S^T and would otherwise expose a memory round trip
    f32x4 u0n[CT];
#pragma unroll
    for (int jt = 0; jt < CT; ++jt) u0n[jt] = zf4();
    auto load_u0 = [&](int cr) {
        const int c = cr < NC ? cr : NC - 1;
        const float* un = p.ws.u + ((static_cast<int64_t>(bh) * NC + c) * DV + v0 + r16) * C + 4 * g;
#pragma unroll
        for (int jt = 0; jt < CT; ++jt) u0n[jt] = ldf4(un + 16 * jt);
    };

    if (NC > 0) {
        if (kh == 0) load_u0(0);
        fetch(0);
        stage(0, 0);
        fetch(1);
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            const int b = c & 1;
            const int64_t chunk = static_cast<int64_t>(bh) * NC + c;

            // ---- phase 1
            f32x4 u0[CT];
#pragma unroll
            for (int jt = 0; jt < CT; ++jt) u0[jt] = u0n[jt];
            if (kh == 0) load_u0(c + 1);
            u16* const st = p.ws.s + (chunk * DV + v0 + r16) * DK + key0 + 4 * g;
#pragma unroll
            for (int t = 0; t < KTW; ++t) st4(st + 16 * t, cvt4(sacc[t]));
            // y[jt][r] for token 16jt + 4g + r of value v0 + r16: U0 - (W S^T) over this wave's keys
            f32x4 y[CT];
            const u16* w_ = sW(b);
#pragma unroll
            for (int jt = 0; jt < CT; ++jt) {
                f32x4 acc = zf4();
                if constexpr (KTW == 1) {
                    const u16* wr = w_ + (16 * jt + r16) * WS + key0 + 4 * g;
                    acc = mfma_16x16x32(join8(ld4(wr), zero4()), join8(cvt4(sacc[0]), zero4()), acc);
                } else {
#pragma unroll
                    for (int kb = 0; kb < KTW / 2; ++kb) {
                        const u16* wr = w_ + (16 * jt + r16) * WS + key0 + 32 * kb + 4 * g;
                        acc = mfma_16x16x32(join8(ld4(wr), ld4(wr + 16)),
                                            join8(cvt4(sacc[2 * kb]), cvt4(sacc[2 * kb + 1])), acc);
                    }
                }
                y[jt] = (kh == 0) ? u0[jt] - acc : -acc;
            }
            if constexpr (NKH > 1) {
                float* const mine = sX + ((vt * NKH + kh) * 16 + r16) * XS;
#pragma unroll
                for (int jt = 0; jt < CT; ++jt) stf4(mine + 16 * jt + 4 * g, y[jt]);
            }
            lds_barrier();

            // ---- phase 2
            f32x4 U[CT];
#pragma unroll
            for (int jt = 0; jt < CT; ++jt) U[jt] = y[jt];
            if constexpr (NKH > 1) {
#pragma unroll
                for (int o = 1; o < NKH; ++o) {
                    const float* other = sX + ((vt * NKH + (kh + o) % NKH) * 16 + r16) * XS;
#pragma unroll
                    for (int jt = 0; jt < CT; ++jt) U[jt] = U[jt] + ldf4(other + 16 * jt + 4 * g);
                }
            }
            // carry: weights e^(G_last - G_j); padded tokens have U = 0 and a flat G
            const float* g_ = sG(b);
            const float glast = g_[C - 1];
            const float dec = ex2(glast);
            bf16x4 ub[CT];
#pragma unroll
            for (int jt = 0; jt < CT; ++jt) {
                const f32x4 gj = ldf4(g_ + 16 * jt + 4 * g);
                f32x4 wu;
#pragma unroll
                for (int e = 0; e < 4; ++e) wu[e] = U[jt][e] * ex2(glast - gj[e]);
                ub[jt] = cvt4(wu);
            }
            const u16* k_ = sK(b);
#pragma unroll
            for (int t = 0; t < KTW; ++t) {
                f32x4 acc = sacc[t] * dec;
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    const bool hi = 2 * jb + 1 < CT;
                    acc = mfma_16x16x32(tr_split<KS>(k_, jb, key0 + 16 * t, hi, r16, g),
                                        join8(ub[2 * jb], hi ? ub[(2 * jb + 1) % CT] : zero4()), acc);
                }
                sacc[t] = acc;
            }
            if (c + 1 < NC) stage(b ^ 1, c + 1);
            fetch(c + 2);
            lds_barrier();
        }
    }

    if (p.s_out) {
        float* so = p.s_out + (static_cast<int64_t>(bh) * DV + v0 + r16) * DK + key0 + 4 * g;
#pragma unroll
        for (int t = 0; t < KTW; ++t) stf4(so + 16 * t, sacc[t]);
    }
}

// ====================================================================== output
//
// One workgroup (four waves) per (sequence, chunk); the same shape as the output
// pass of retention: P tiles spread over the waves and shared in LDS, each wave a
// pair of 16-channel value tiles, the readout with S rows from registers - here
// scaled by e^(G_i) - plus P U. U^T rows start as U0 from the workspace; W takes
// the place of k in LDS once P is formed, and W S_in^T (the S rows again as the B
// operand) is subtracted in the accumulator layout of those rows. U enters P U as
// a bf16 hi + lo pair.
template <int C, int DK, int DV>
struct DOutLayout {
    static constexpr int QS = tile_stride(DK);   // rows 8 banks apart: conflict-free 16-byte row reads
    static constexpr int PS = C + 4;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + al(C * QS * 2);
    static constexpr int oP = oK + al(C * QS * 2);
    static constexpr int oG = oP + al(C * PS * 2);
    static constexpr int NP = DV >= 32 ? DV / 32 : 1;
    static constexpr int oR = oG + al(C * 4);            // RMS norm: per (value pair, row) partial sums
    static constexpr int bytes = oR + al(NP * C * 4);
    static_assert(bytes <= 64 * 1024, "LDS budget of the delta output pass exceeded");
};

template <int C, int DK, int DV>
__global__ __launch_bounds__(256)
void delta_output_kernel(DeltaParams p) {
    using Lay = DOutLayout<C, DK, DV>;
    constexpr int NW = 4, NT = 256;
    constexpr int CT = C / 16, JB = (CT + 1) / 2;
    constexpr int KB = (DK + 31) / 32;
    constexpr int QS = Lay::QS, PS = Lay::PS;
    constexpr int QP = C * DK / 8, QP_PER = (QP + NT - 1) / NT;
    constexpr int NP = DV >= 32 ? DV / 32 : 1;
    static_assert(NW % NP == 0, "waves must cover the value pairs evenly");
    constexpr int NPAIR = CT * (CT + 1) / 2;

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sQ = reinterpret_cast<u16*>(smem + Lay::oQ);
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    u16* const sP = reinterpret_cast<u16*>(smem + Lay::oP);
    float* const sG = reinterpret_cast<float*>(smem + Lay::oG);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
    const int T = p.T;
    const int t0 = c * C, n = (T - t0 < C) ? (T - t0) : C;
    const int64_t tok0 = static_cast<int64_t>(bh) * T + t0;
    const int64_t chunk = static_cast<int64_t>(bh) * p.NC + c;
    const u16* sc = p.ws.s + chunk * DV * DK;
    const float* uc = p.ws.u + chunk * DV * C;
    const u16* wc = p.ws.w + chunk * C * DK;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};

    // ---- loads up front: q, k, W pieces; this wave's S rows and U0^T rows
    u16x8 rq[QP_PER], rk[QP_PER], rw[QP_PER];
#pragma unroll
    for (int i = 0; i < QP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        const unsigned off = (idx < QP && j < n) ? static_cast<unsigned>(j * DK + col) : 0u;
        rq[i] = *reinterpret_cast<const u16x8*>(p.q + tok0 * DK + off);
        rk[i] = *reinterpret_cast<const u16x8*>(((p.fuse & 1) ? p.ws.kn + chunk * C * DK : p.k + tok0 * DK) + off);
        rw[i] = *reinterpret_cast<const u16x8*>(wc + off);
    }
    const float gl = (tid < C) ? p.ws.g[chunk * C + tid] : 0.f;
    const int pp = w % NP;
    u16x8 sa[2][KB];
    f32x4 ua[2][JB][2];   // U0^T (later U^T) rows: [tile][jb][half], tokens 32jb + 16 half + 4g + e
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int vrow = (DV >= 32) ? 32 * pp + 16 * tt + r16 : r16;
        const bool live = DV >= 32 || tt == 0;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            sa[tt][kb] = (live && col < DK) ? *reinterpret_cast<const u16x8*>(sc + vrow * DK + col) : z8;
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int j0 = 32 * jb + 16 * hf + 4 * g;
                ua[tt][jb][hf] = (live && j0 < C) ? ldf4(uc + vrow * C + j0) : zf4();
            }
    }

    // ---- stage q, k, G
#pragma unroll
    for (int i = 0; i < QP_PER; ++i) {
        const int idx = tid + i * NT;
        const u16x8 qx = (p.fuse & 1) ? silu_l2_piece<DK / 8>(rq[i]) : rq[i];
        const u16x8 kx = rk[i];   // mapped by the prep when the feature map is fused
        if (idx < QP) {
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const bool ok = j < n;
            *reinterpret_cast<u16x8*>(sQ + j * QS + col) = ok ? qx : z8;
            *reinterpret_cast<u16x8*>(sK + j * QS + col) = ok ? kx : z8;
        }
    }
    if (tid < C) sG[tid] = gl;
    lds_barrier();

    // ---- P tiles: P_ij = (q_i . k_j) e^(G_i - G_j), j <= i
    for (int pr0 = w; pr0 < NPAIR; pr0 += NW) {
        int it = 0, jt = pr0;
        while (jt > it) { jt -= it + 1; ++it; }
        const int i = 16 * it + r16;
        f32x4 acc = zf4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            bf16x8 ka = as_bf16x8(z8), qb = as_bf16x8(z8);
            if (col < DK) {
                ka = *reinterpret_cast<const bf16x8*>(sK + (16 * jt + r16) * QS + col);
                qb = *reinterpret_cast<const bf16x8*>(sQ + i * QS + col);
            }
            acc = mfma_16x16x32(ka, qb, acc);
        }
        const float gi = sG[i];
        const f32x4 gj = ldf4(sG + 16 * jt + 4 * g);
        bf16x4 pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * g + r;
            pv[r] = static_cast<__bf16>((j <= i) ? acc[r] * ex2(fminf(gi - gj[r], 0.f)) : 0.f);
        }
        st4(sP + i * PS + 16 * jt + 4 * g, pv);
    }
    lds_barrier();

    // ---- U = U0 - W S_in^T: W over k in LDS, then per value tile and token tile
    // D[token 4g + r][value r16] += W[token][keys] S[value][keys]
#pragma unroll
    for (int i = 0; i < QP_PER; ++i) {
        const int idx = tid + i * NT;
        if (idx < QP) {
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            *reinterpret_cast<u16x8*>(sK + j * QS + col) = (j < n) ? rw[i] : z8;
        }
    }
    lds_barrier();
#pragma unroll
    for (int tt = 0; tt < (DV >= 32 ? 2 : 1); ++tt) {
#pragma unroll
        for (int jt = 0; jt < CT; ++jt) {
            f32x4 acc = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int col = 32 * kb + 8 * g;
                const bf16x8 wa = (col < DK) ? *reinterpret_cast<const bf16x8*>(sK + (16 * jt + r16) * QS + col)
                                             : as_bf16x8(z8);
                acc = mfma_16x16x32(wa, as_bf16x8(sa[tt][kb]), acc);
            }
            ua[tt][jt >> 1][jt & 1] = ua[tt][jt >> 1][jt & 1] - acc;
        }
    }

    // ---- outputs: e^(G_i) S_in q_i + P U, items (row tile, value pair) kept in registers
    // until the optional RMS norm has every row's sum of squares
    constexpr int ITEMS = (CT * NP + NW - 1) / NW;
    f32x4 ov[ITEMS][2];
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
        const int item = w + NW * s;
        ov[s][0] = zf4();
        ov[s][1] = zf4();
        if (item >= CT * NP) continue;
        const int it = item / NP;
        const int i = 16 * it + r16;
        const float oscale = ex2(sG[i]);
        bf16x8 qb[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            qb[kb] = (col < DK) ? *reinterpret_cast<const bf16x8*>(sQ + i * QS + col) : as_bf16x8(z8);
        }
        bf16x8 pb[JB];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            if (2 * jb <= it) {
                const u16* prow = sP + i * PS + 32 * jb + 4 * g;
                pb[jb] = join8(ld4(prow), (2 * jb + 1 <= it) ? ld4(prow + 16) : zero4());
            }
        }
#pragma unroll
        for (int tt = 0; tt < (DV >= 32 ? 2 : 1); ++tt) {
            f32x4 acc = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc = mfma_16x16x32(as_bf16x8(sa[tt][kb]), qb[kb], acc);
            acc = acc * oscale;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if (2 * jb <= it) {
                    const bool hi = 2 * jb + 1 <= it;
                    const f32x4 u0 = ua[tt][jb][0];
                    const f32x4 u1 = hi ? ua[tt][jb][1] : zf4();
                    const bf16x4 h0 = cvt4(u0), h1 = cvt4(u1);
                    acc = mfma_16x16x32(join8(h0, h1), pb[jb], acc);
                    acc = mfma_16x16x32(join8(cvt4(u0 - up4(h0)), cvt4(u1 - up4(h1))), pb[jb], acc);
                }
            }
            ov[s][tt] = acc;
        }
    }
    if (p.fuse & 2) {
        // lane (r16, g) of item (it, pp) holds o[16it + r16][32pp + 16tt + 4g + r]: the
        // pair's share of each row's sum of squares, over g by shuffles, then over the
        // pairs in LDS
        float* const sRow = reinterpret_cast<float*>(smem + Lay::oR);
#pragma unroll
        for (int s = 0; s < ITEMS; ++s) {
            const int item = w + NW * s;
            float ss = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) ss += ov[s][tt][r] * ov[s][tt][r];
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            if (item < CT * NP && g == 0) sRow[pp * C + 16 * (item / NP) + r16] = ss;
        }
        lds_barrier();
#pragma unroll
        for (int s = 0; s < ITEMS; ++s) {
            const int item = w + NW * s;
            if (item >= CT * NP) continue;
            const int i = 16 * (item / NP) + r16;
            float tot = 0.f;
#pragma unroll
            for (int q2 = 0; q2 < NP; ++q2) tot += sRow[q2 * C + i];
            const float inv = 1.f / __builtin_sqrtf(tot / static_cast<float>(DV) + p.oeps);
#pragma unroll
            for (int tt = 0; tt < (DV >= 32 ? 2 : 1); ++tt) {
                const f32x4 wv = ldf4(p.onw + ((DV >= 32) ? 32 * pp + 16 * tt : 0) + 4 * g);
                ov[s][tt] = ov[s][tt] * wv * inv;
            }
        }
    }
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
        const int item = w + NW * s;
        if (item >= CT * NP) continue;
        const int i = 16 * (item / NP) + r16;
        if (i < n) {
            u16* orow = p.o + (tok0 + i) * DV;
            if constexpr (DV >= 32) {
                st4(orow + 32 * pp + 4 * g, cvt4(ov[s][0]));
                st4(orow + 32 * pp + 16 + 4 * g, cvt4(ov[s][1]));
            } else {
                st4(orow + 4 * g, cvt4(ov[s][0]));
            }
        }
    }
}

// ====================================================================== launch
template <int C, int DK, int DV>
hipError_t launch_delta_dv(const ChunkArgs& a, hipStream_t stream) {
    const int NC = (a.T + C - 1) / C;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    DeltaParams p{};
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.alpha = a.gate;
    p.beta = a.beta;
    p.s0 = a.s0;
    p.o = static_cast<u16*>(a.o);
    p.s_out = a.s_out;
    p.ws = delta_ws_split(a.ws, heads * NC, C, DK, DV);
    p.T = a.T;
    p.NC = NC;
    p.fuse = a.fuse;
    p.onw = a.onw;
    p.oeps = a.oeps;
    // state pass: two value tiles x two key groups per workgroup (fewer when the head is small)
    constexpr int NVT = DV >= 32 ? 2 : 1;
    constexpr int NKH = DK >= 32 ? 2 : 1;
    p.vblocks = DV / (16 * NVT);
    if (NC > 0) {
        hipLaunchKernelGGL((delta_prep_kernel<C, DK, DV>), dim3(static_cast<unsigned>(heads * NC)), dim3(256), 0,
                           stream, p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((delta_state_kernel<C, DK, DV, NVT, NKH>), dim3(static_cast<unsigned>(heads * p.vblocks)),
                       dim3(64 * NVT * NKH), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || NC == 0) return err;
    hipLaunchKernelGGL((delta_output_kernel<C, DK, DV>), dim3(static_cast<unsigned>(heads * NC)), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

template <int C, int DK>
hipError_t launch_delta_dk(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_delta_dv<C, DK, 16>(a, stream);
        case 32: return launch_delta_dv<C, DK, 32>(a, stream);
        case 64: return launch_delta_dv<C, DK, 64>(a, stream);
        case 128: return launch_delta_dv<C, DK, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int C>
hipError_t launch_delta(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_delta_dk<C, 16>(a, stream);
        case 32: return launch_delta_dk<C, 32>(a, stream);
        case 64: return launch_delta_dk<C, 64>(a, stream);
        case 128: return launch_delta_dk<C, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
