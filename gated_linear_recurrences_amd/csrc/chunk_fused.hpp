// Single-pass chunked forward for retention and the scalar data-dependent decay (bf16
// storage): the memory never leaves the chip. Chunks 16 and 32 and d_k = 16; chunk 64 with
// d_k >= 32 takes the gated delta rule's single pass without its delta step
// (chunk_delta_sp.hpp).
//
// Method: the chunkwise form of retention ("Le architetture lineari: RetNet, RWKV,
// xLSTM", section "RetNet: la retention e le sue tre forme", Fig. 16.5) and its
// scalar data-dependent gate ("Scrivere meglio nella memoria", section "Dimenticare: i
// gate", the scalar decay). With local index i, j, n tokens in the chunk, the memory
// S_in entering it and G the chunk-local inclusive cumulative log-gate (retention:
// G_i = (i + 1) log g):
//   o_i   = sum_{j<=i} e^(G_i - G_j) (q_i . k_j) v_j + e^(G_i) S_in q_i
//   S_out = e^(G_{n-1}) S_in + sum_j e^(G_{n-1} - G_j) v_j k_j^T
// Rows of S (value channels) evolve independently, so a workgroup owns one sequence and
// a slice of 16 TS value channels, and walks the chunks in order with its slice of S in
// fp32 MFMA accumulators: no snapshot of S goes to HBM, and each chunk's output is
// produced as soon as its S_in is known. The workgroups of one sequence (the slices)
// run side by side on one XCD and share q and k through its L2.
//
// Decomposition (gfx950), four waves, per chunk:
//   operands  k, the v slice (and the raw scalar gates) are staged in LDS
//             (double-buffered), loaded two chunks ahead through a two-slot register ring
//             that is written to LDS just before the chunk's barrier: every load is
//             consumed there, so the compiler's count of loads in flight stays exact and
//             one chunk's loads stay in flight across each wait. q is staged the same way
//             at chunks 16 and 32; at chunk 64 each wave loads its own 16 rows of q into
//             the ring, in the MFMA operand layout, and takes them from there;
//   gates     retention's decay factors depend only on positions: they are tabulated in
//             registers once. For the scalar gate every wave scans the chunk's raw gates
//             and tabulates e^(G), e^(-G) and the carry weights e^(G_last - G) in its own
//             LDS rows (one exponential per lane per table), so that e^(G_i - G_j) is a
//             product of two table entries;
//   triangle  wave w forms P[i][j] = (q_i . k_j) e^(G_i - G_j), i in tile w, j <= i, one
//             MFMA chain over d_k per 16 x 16 tile; all of the wave's LDS operands are
//             requested before its independent chains run interleaved (one wave per SIMD:
//             nothing else hides the LDS latency). P stays in registers, already in the
//             operand layout of P V;
//   output    o^T = e^(G_i) S_in q^T (S_in read from LDS as bf16 rows) + V^T P^T, V^T
//             read by ds_read_b64_tr_b16; each lane holds four consecutive value channels
//             of one token, stored after the staging;
//   carry     wave w owns key tiles w, w + 4, ... of S^T: S^T <- e^(G_last) S^T +
//             K^T diag(wt) V, the weights applied to the V operand already read for the
//             output; the new memory goes to the other bf16 LDS buffer as the next
//             chunk's readout operand.
// One workgroup barrier per chunk.
#pragma once

#include <type_traits>

#include "chunk_common.hpp"

namespace glr {
namespace ck {

struct FusedParams {
    const u16* q;        // [BH][T][DK]
    const u16* k;        // [BH][T][DK]
    const u16* v;        // [BH][T][DV]
    const float* gate;   // retention: log gamma [H]; scalar: log alpha [BH][T]
    const float* s0;     // [BH][DV][DK] or null
    u16* o;              // [BH][T][DV]
    float* s_out;        // [BH][DV][DK] or null
    int H, T, NC, slices, remap;
};

template <int C, int DK, int DVS, int GK>
struct FusedLayout {
    using TK = SwzTile<DK>;
    using TV = SwzTile<DVS>;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int KBUF = al(C * TK::STRIDE * 2);     // q or k, token-major
    static constexpr int VBUF = al(C * TV::STRIDE * 2);     // v slice, token-major
    static constexpr int SBUF = al(DVS * TK::STRIDE * 2);   // S_in slice, bf16 rows
    static constexpr int GBUF = GK == kGateScalar ? al(C * 4) : 0;
    // with four token tiles every wave reads only its own 16 rows of q: they go from HBM
    // straight to its registers, and only k, v (and the gates) are staged
    static constexpr bool QREG = C == 64;
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + (QREG ? 0 : 2 * KBUF);
    static constexpr int oV = oK + 2 * KBUF;
    static constexpr int oS = oV + 2 * VBUF;
    static constexpr int oG = oS + 2 * SBUF;
    // per-wave gate tables: scalar, 4 rows of C floats; fixed, the per-lane decay factors of
    // the triangle tiles and the carry weights (f32x4 per lane)
    static constexpr int CT = C / 16, JB = (CT + 1) / 2;
    static constexpr int TABW = GK == kGateScalar ? 4 * C * 4 : (CT + 2 * JB) * 64 * 16;
    static constexpr int oT = oG + 2 * GBUF;
    static constexpr int bytes = oT + 4 * TABW;
    static_assert(bytes <= 160 * 1024, "LDS budget of the single-pass forward exceeded");
};

template <int C, int DK, int DV, int TS, int GK>
__global__ __launch_bounds__(256)
void fused_kernel(FusedParams p) {
    constexpr int DVS = 16 * TS;
    using Lay = FusedLayout<C, DK, DVS, GK>;
    using TK = SwzTile<DK>;
    constexpr bool SCL = GK == kGateScalar;
    constexpr int NT = 256;
    constexpr int CT = C / 16;                 // token tiles (waves w < CT own one each)
    constexpr int KB = (DK + 31) / 32;         // 32-wide blocks of d_k
    constexpr int NKT = DK / 16;               // key tiles of S^T
    constexpr int KTW = (NKT + 3) / 4;         // key tiles per wave
    constexpr int JB = (CT + 1) / 2;           // 32-token blocks
    constexpr int KP = C * DK / 8, KP_PER = (KP + NT - 1) / NT;     // 16-byte pieces of k
    // pieces of the v slice: 8 bytes when that gives every thread exactly one
    constexpr int VE = (C * DVS / 4 == NT) ? 4 : 8;                 // elements per piece
    constexpr int VP = C * DVS / VE, VP_PER = (VP + NT - 1) / NT;
    static_assert(DV % DVS == 0, "value slices must tile d_v");
    constexpr bool QREG = Lay::QREG;
    constexpr int QN = QREG ? KB : KP_PER;     // q pieces per lane and chunk

    __shared__ __align__(16) unsigned char smem[Lay::bytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;

    const int lb = logical_block_of(blockIdx.x, gridDim.x, p.remap);
    const int bh = lb / p.slices, m0 = (lb % p.slices) * DVS;
    const int T = p.T, NC = p.NC;
    const int64_t seq0 = static_cast<int64_t>(bh) * T;
    const u16* qs = p.q + seq0 * DK;
    const u16* ks = p.k + seq0 * DK;
    const u16* vs = p.v + seq0 * DV + m0;
    u16* os = p.o + seq0 * DV + m0;
    const float* gs = SCL ? p.gate + seq0 : nullptr;
    const float lg2 = SCL ? 0.f : p.gate[bh % p.H] * kLog2e;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};

    auto sQ = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oQ + b * Lay::KBUF); };
    auto sK = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oK + b * Lay::KBUF); };
    auto sV = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oV + b * Lay::VBUF); };
    auto sS = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oS + b * Lay::SBUF); };
    auto sG = [&](int b) { return reinterpret_cast<float*>(smem + Lay::oG + b * Lay::GBUF); };
    auto count = [&](int c) { return (T - c * C < C) ? (T - c * C) : C; };

    // ---- register ring: q, k and v pieces (and the raw gates) of two chunks
    typedef unsigned short vpiece __attribute__((ext_vector_type(VE)));
    u16x8 rq[2][QN], rk[2][KP_PER];
    vpiece rv[2][VP_PER];
    float rg[2];

    // Loads are issued by every lane without branches (indices clamped, values past the end
    // zeroed when staged) and consumed only when staged, so that the compiler's count of
    // loads in flight stays exact across the chunk loop and each wait covers only the chunk
    // it is for.
    auto load = [&](int c, u16x8 (&q)[QN], u16x8 (&k)[KP_PER], vpiece (&v)[VP_PER], float& gr) {
        const int n = count(c);
        const int64_t t0 = static_cast<int64_t>(c) * C;
        if constexpr (QREG) {
            // row 16w + r16 in the operand layout of the products over d_k (pieces rr_col);
            // rows past the end reload row 0: they only reach outputs that are not stored.
            // Issued first, so the wait before the next staging covers them too.
            const int i = 16 * w + r16;
            const int64_t row = t0 + (i < n ? i : 0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int col = rr_col(kb, g, KB);
                q[kb] = *reinterpret_cast<const u16x8*>(qs + row * DK + (col < DK ? col : 0));
            }
        }
#pragma unroll
        for (int i = 0; i < KP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const int64_t off = (t0 + ((idx < KP && j < n) ? j : 0)) * DK + (idx < KP ? col : 0);
            if constexpr (!QREG) q[i] = *reinterpret_cast<const u16x8*>(qs + off);
            k[i] = *reinterpret_cast<const u16x8*>(ks + off);
        }
#pragma unroll
        for (int i = 0; i < VP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DVS / VE), col = (idx % (DVS / VE)) * VE;
            const int jj = (idx < VP && j < n) ? j : 0;
            v[i] = *reinterpret_cast<const vpiece*>(vs + (t0 + jj) * DV + (idx < VP ? col : 0));
        }
        if constexpr (SCL) gr = gs[t0 + (lane < n ? lane : 0)];   // zeroed past the end when staged
    };
    auto stage = [&](int c, int b, const u16x8 (&q)[QN], const u16x8 (&k)[KP_PER], const vpiece (&v)[VP_PER],
                     float gr) {
        const int n = count(c);
        u16* Q = sQ(b);
        u16* K = sK(b);
        u16* V = sV(b);
#pragma unroll
        for (int i = 0; i < KP_PER; ++i) {
            const int idx = tid + i * NT;
            // no branch when the pieces cover the threads evenly (every staged register is
            // consumed on every path)
            if (KP % NT == 0 || idx < KP) {
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                if constexpr (!QREG) *reinterpret_cast<u16x8*>(Q + TK::off(j, col)) = j < n ? q[i] : z8;
                *reinterpret_cast<u16x8*>(K + TK::off(j, col)) = j < n ? k[i] : z8;
            }
        }
#pragma unroll
        for (int i = 0; i < VP_PER; ++i) {
            const int idx = tid + i * NT;
            if (VP % NT == 0 || idx < VP) {
                const int j = idx / (DVS / VE), col = (idx % (DVS / VE)) * VE;
                const vpiece zv = {};
                *reinterpret_cast<vpiece*>(V + SwzTile<DVS>::off(j, col)) = j < n ? v[i] : zv;
            }
        }
        if constexpr (SCL) {
            // raw gates (past the end: 0); every wave writes its copy, so that the loaded
            // gates are consumed on every path
            if (lane < C) sG(b)[lane] = lane < n ? gr : 0.f;
        }
    };

    float* const tab = reinterpret_cast<float*>(smem + Lay::oT + w * Lay::TABW);   // this wave's gate tables
    f32x4* const tabl = reinterpret_cast<f32x4*>(tab) + lane;   // fixed gate: entry e at tabl[64 e]

    // ---- this wave's key tiles of S^T (fp32): sacc[u][tt][r] = S[m0 + 16tt + r16][16kt + 4g + r]
    f32x4 sacc[KTW][TS];
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
        const int kt = w + 4 * u;
#pragma unroll
        for (int tt = 0; tt < TS; ++tt) {
            sacc[u][tt] = zf4();
            if (kt < NKT && p.s0 != nullptr)
                sacc[u][tt] = ldf4(p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * tt + r16) * DK + 16 * kt + 4 * g);
            if (kt < NKT) st4(sS(0) + TK::off(16 * tt + r16, 16 * kt + 4 * g), cvt4(sacc[u][tt]));
        }
    }

    // ---- fixed gate: decay factors by position, tabulated once in this wave's LDS rows
    // (entries 0..CT-1: the triangle tiles of row tile w; then the carry weights of each
    // 32-token block, low and high half, for a full chunk)
    auto carry_weight = [&](int j, int n) { return j < n ? ex2(static_cast<float>(n - 1 - j) * lg2) : 0.f; };
    float osc = 0.f;
    if constexpr (!SCL) {
        const int i = 16 * w + r16;
#pragma unroll
        for (int jt = 0; jt < CT; ++jt) {
            f32x4 d;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 16 * jt + 4 * g + r;
                d[r] = j <= i ? ex2(static_cast<float>(i - j) * lg2) : 0.f;
            }
            tabl[64 * jt] = d;
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            f32x4 lo, hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo[e] = carry_weight(32 * jb + 4 * g + e, C);
                hi[e] = carry_weight(32 * jb + 16 + 4 * g + e, C);
            }
            tabl[64 * (CT + 2 * jb)] = lo;
            tabl[64 * (CT + 2 * jb + 1)] = hi;
        }
        osc = ex2(static_cast<float>(i + 1) * lg2);
    }

    if (NC > 0) {
        load(0, rq[0], rk[0], rv[0], rg[0]);
        load(NC > 1 ? 1 : 0, rq[1], rk[1], rv[1], rg[1]);
        stage(0, 0, rq[0], rk[0], rv[0], rg[0]);
    }
    lds_barrier();

    // One chunk as wave W (a compile-time role: token tile W's outputs when W < CT, key tiles
    // W, W + 4, ... of the carry).
    auto compute = [&](int c, const u16* Qc, const u16* K, const u16* V, const u16* Sin, u16* Snext,
                       const float* graw, bf16x4 (&ov)[TS], auto wrole, auto&& issue_loads,
                       const u16x8 (&qr)[QN]) __attribute__((always_inline)) {
        constexpr int W = decltype(wrole)::value;
        constexpr int NJ = W < CT ? W + 1 : 0;      // P tiles of this wave's row tile
        constexpr int NJA = NJ > 0 ? NJ : 1;
        constexpr int NU = (NKT > W) ? (NKT - W + 3) / 4 : 0;   // carry key tiles
        constexpr int NUA = NU > 0 ? NU : 1;
        const int n = count(c);
        const int i = 16 * W + r16;

        // ---- operand reads
        bf16x8 qb[KB], kr[NJA][KB], sa[TS][KB];
        bf16x4 vl[TS][JB], vh[TS][JB], kl[NUA][JB], kh[NUA][JB];
        if constexpr (NJ > 0) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int col = rr_col(kb, g, KB);
                const bool in = col < DK;
                if constexpr (QREG)
                    qb[kb] = in ? as_bf16x8(qr[kb]) : as_bf16x8(z8);
                else
                    qb[kb] = in ? *reinterpret_cast<const bf16x8*>(Qc + TK::off(i, col)) : as_bf16x8(z8);
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt)
                    kr[jt][kb] = in ? *reinterpret_cast<const bf16x8*>(K + TK::off(16 * jt + r16, col)) : as_bf16x8(z8);
#pragma unroll
                for (int tt = 0; tt < TS; ++tt)
                    sa[tt][kb] = in ? *reinterpret_cast<const bf16x8*>(Sin + TK::off(16 * tt + r16, col)) : as_bf16x8(z8);
            }
        }
#pragma unroll
        for (int tt = 0; tt < TS; ++tt)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                vl[tt][jb] = tr_op_s<DVS>(V, 32 * jb, 16 * tt, r16, g);
                vh[tt][jb] = (32 * jb + 16 < C) ? tr_op_s<DVS>(V, 32 * jb + 16, 16 * tt, r16, g) : zero4();
            }
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                kl[u][jb] = tr_op_s<DK>(K, 32 * jb, 16 * (W + 4 * u), r16, g);
                kh[u][jb] = (32 * jb + 16 < C) ? tr_op_s<DK>(K, 32 * jb + 16, 16 * (W + 4 * u), r16, g) : zero4();
            }

        // the loads of chunk c + 2 go out while these reads are in flight: a CU's address
        // unit takes about 64 bytes of loads per cycle, so issuing a chunk's loads (9 per
        // lane) stalls the wave for hundreds of cycles, hidden here behind the LDS latency
        issue_loads();

        // ---- scalar gate: inclusive scan of the raw gates (log2 units; padded tokens add 0),
        // then this wave's tables: G, e^G, e^-G and the carry weights e^(G_last - G) (0 past
        // the end), read back just before their products
        float Gl = 0.f;
        if constexpr (SCL) {
            const float x = (lane < n) ? graw[lane] * kLog2e : 0.f;
            const float G = wave_inclusive_scan(x);
            Gl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), C - 1));
            if (lane < C) {
                tab[lane] = G;
                tab[C + lane] = ex2(G);
                tab[2 * C + lane] = ex2(-G);
                tab[3 * C + lane] = lane < n ? ex2(Gl - G) : 0.f;
            }
        }

        // ---- triangle and readout: independent chains, interleaved over d_k
        f32x4 pacc[NJA], oacc[TS];
#pragma unroll
        for (int jt = 0; jt < NJA; ++jt) pacc[jt] = zf4();
#pragma unroll
        for (int tt = 0; tt < TS; ++tt) oacc[tt] = zf4();
        if constexpr (NJ > 0) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) pacc[jt] = mfma_16x16x32(kr[jt][kb], qb[kb], pacc[jt]);
#pragma unroll
                for (int tt = 0; tt < TS; ++tt) oacc[tt] = mfma_16x16x32(sa[tt][kb], qb[kb], oacc[tt]);
            }

            // ---- decay factors of the triangle (the diagonal tile masked above the diagonal)
            f32x4 dq[NJA];
            float oscale;
            if constexpr (SCL) {
                oscale = tab[C + i];
                if (Gl >= -100.f) {
                    // e^(G_i - G_j) = e^(G_i) e^(-G_j): both factors within 2^+-100
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) dq[jt] = ldf4(tab + 2 * C + 16 * jt + 4 * g) * oscale;
                } else {
                    const float Gi = tab[i];
#pragma unroll
                    for (int jt = 0; jt < NJ; ++jt) {
                        const f32x4 Gj = ldf4(tab + 16 * jt + 4 * g);
#pragma unroll
                        for (int r = 0; r < 4; ++r) dq[jt][r] = ex2(Gi - Gj[r]);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (16 * (NJ - 1) + 4 * g + r > i) dq[NJ - 1][r] = 0.f;
            } else {
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) dq[jt] = tabl[64 * jt];
                oscale = osc;
            }

            // ---- output: o^T = e^(G_i) S_in q^T + V^T P^T
            bf16x8 pb[JB];
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
                if (2 * jb < NJ)
                    pb[jb] = join8(cvt4(pacc[2 * jb] * dq[2 * jb]),
                                   2 * jb + 1 < NJ ? cvt4(pacc[2 * jb + 1] * dq[2 * jb + 1]) : zero4());
#pragma unroll
            for (int tt = 0; tt < TS; ++tt) {
                f32x4 acc = oacc[tt] * oscale;
#pragma unroll
                for (int jb = 0; jb < JB; ++jb)
                    if (2 * jb < NJ) acc = mfma_16x16x32(join8(vl[tt][jb], vh[tt][jb]), pb[jb], acc);
                ov[tt] = cvt4(acc);   // o[i][m0 + 16tt + 4g + r], stored after the staging
            }
        }

        // ---- carry: S^T <- e^(G_last) S^T + K^T diag(wt) V; the new S_in for the readout
        if constexpr (NU > 0) {
            f32x4 cwl[JB], cwh[JB];
            float cdecay;
            if constexpr (SCL) {
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    cwl[jb] = ldf4(tab + 3 * C + 32 * jb + 4 * g);
                    cwh[jb] = (32 * jb + 16 < C) ? ldf4(tab + 3 * C + 32 * jb + 16 + 4 * g) : zf4();
                }
                cdecay = ex2(Gl);
            } else if (n == C) {
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    cwl[jb] = tabl[64 * (CT + 2 * jb)];
                    cwh[jb] = tabl[64 * (CT + 2 * jb + 1)];
                }
                cdecay = ex2(static_cast<float>(C) * lg2);
            } else {
                // a short last chunk
#pragma unroll
                for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        cwl[jb][e] = carry_weight(32 * jb + 4 * g + e, n);
                        cwh[jb][e] = carry_weight(32 * jb + 16 + 4 * g + e, n);
                    }
                cdecay = ex2(static_cast<float>(n) * lg2);
            }
            bf16x8 vw[TS][JB];
#pragma unroll
            for (int tt = 0; tt < TS; ++tt)
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) vw[tt][jb] = join8(scale4(vl[tt][jb], cwl[jb]), scale4(vh[tt][jb], cwh[jb]));
#pragma unroll
            for (int u = 0; u < NU; ++u) {
#pragma unroll
                for (int tt = 0; tt < TS; ++tt) {
                    f32x4 acc = sacc[u][tt] * cdecay;
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) acc = mfma_16x16x32(join8(kl[u][jb], kh[u][jb]), vw[tt][jb], acc);
                    sacc[u][tt] = acc;
                    st4(Snext + TK::off(16 * tt + r16, 16 * (W + 4 * u) + 4 * g), cvt4(acc));
                }
            }
        }
    };

    // one chunk; slot S = c & 1 names both the register slot and the LDS buffer
    auto step = [&](int c, auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        // past the end: a harmless reload
        auto issue_loads = [&]() __attribute__((always_inline)) {
            load((c + 2 < NC) ? c + 2 : NC - 1, rq[S], rk[S], rv[S], rg[S]);
        };
        const u16 *Qc = sQ(S), *K = sK(S), *V = sV(S), *Sin = sS(S);
        u16* Snext = sS(S ^ 1);
        const float* graw = sG(S);
        bf16x4 ov[TS];
        switch (w) {
            case 0: compute(c, Qc, K, V, Sin, Snext, graw, ov, std::integral_constant<int, 0>{}, issue_loads, rq[S]); break;
            case 1: compute(c, Qc, K, V, Sin, Snext, graw, ov, std::integral_constant<int, 1>{}, issue_loads, rq[S]); break;
            case 2: compute(c, Qc, K, V, Sin, Snext, graw, ov, std::integral_constant<int, 2>{}, issue_loads, rq[S]); break;
            default: compute(c, Qc, K, V, Sin, Snext, graw, ov, std::integral_constant<int, 3>{}, issue_loads, rq[S]); break;
        }
        // ---- next chunk's operands into the other buffer
        // (past the last chunk: a copy of it, never read)
        stage(c + 1 < NC ? c + 1 : c, S ^ 1, rq[S ^ 1], rk[S ^ 1], rv[S ^ 1], rg[S ^ 1]);
        // the outputs go out after the staging: the loads' count of outstanding memory
        // operations (stores included) then does not wait for this store's acknowledgement
        const int i = 16 * w + r16;
        if (w < CT && i < count(c)) {
#pragma unroll
            for (int tt = 0; tt < TS; ++tt) st4(os + (static_cast<int64_t>(c) * C + i) * DV + 16 * tt + 4 * g, ov[tt]);
        }
        lds_barrier();
    };

    // both steps on every trip (an odd last chunk after the loop), so that no path leaves a
    // slot's loads unconsumed at the loop head
    int c = 0;
    for (; c + 1 < NC; c += 2) {
        step(c, std::integral_constant<int, 0>{});
        step(c + 1, std::integral_constant<int, 1>{});
    }
    if (c < NC) step(c, std::integral_constant<int, 0>{});

    if (p.s_out != nullptr) {
#pragma unroll
        for (int u = 0; u < KTW; ++u) {
            const int kt = w + 4 * u;
            if (kt < NKT) {
#pragma unroll
                for (int tt = 0; tt < TS; ++tt)
                    stf4(p.s_out + (static_cast<int64_t>(bh) * DV + m0 + 16 * tt + r16) * DK + 16 * kt + 4 * g,
                         sacc[u][tt]);
            }
        }
    }
}

template <int C, int DK, int DV, int TS, int GK>
hipError_t launch_fused_ts(const ChunkArgs& a, hipStream_t stream) {
    FusedParams p{};
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.gate = a.gate;
    p.s0 = a.s0;
    p.o = static_cast<u16*>(a.o);
    p.s_out = a.s_out;
    p.H = a.H;
    p.T = a.T;
    p.NC = (a.T + C - 1) / C;
    p.slices = DV / (16 * TS);
    const int64_t G = static_cast<int64_t>(a.B) * a.H * p.slices;
    p.remap = (G % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((fused_kernel<C, DK, DV, TS, GK>), dim3(static_cast<unsigned>(G)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// Slices of 32 value channels when that still gives every CU a workgroup, else 16.
template <int C, int DK, int DV, int GK>
hipError_t launch_fused_dv(const ChunkArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if constexpr (DV >= 32) {
        if (heads * (DV / 32) >= kCUs) return launch_fused_ts<C, DK, DV, 2, GK>(a, stream);
    }
    return launch_fused_ts<C, DK, DV, 1, GK>(a, stream);
}

template <int C, int DK, int GK>
hipError_t launch_fused_dk(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_fused_dv<C, DK, 16, GK>(a, stream);
        case 32: return launch_fused_dv<C, DK, 32, GK>(a, stream);
        case 64: return launch_fused_dv<C, DK, 64, GK>(a, stream);
        case 128: return launch_fused_dv<C, DK, 128, GK>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int C, int GK>
hipError_t launch_fused(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_fused_dk<C, 16, GK>(a, stream);
        case 32: return launch_fused_dk<C, 32, GK>(a, stream);
        case 64: return launch_fused_dk<C, 64, GK>(a, stream);
        case 128: return launch_fused_dk<C, 128, GK>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
