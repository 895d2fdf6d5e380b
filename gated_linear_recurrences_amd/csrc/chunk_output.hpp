// Output pass of the two-pass chunked forward for retention, the scalar
// data-dependent decay and GLA (bf16 storage).
//
// Method: the chunkwise form of retention ("Le architetture lineari: RetNet,
// RWKV, xLSTM", section "RetNet: la retention e le sue tre forme", Fig. 16.5)
// and its per-channel gated extension ("Scrivere meglio nella memoria",
// section "Dimenticare: i gate"): inside a chunk the masked decay triangle,
// between chunks the memory. With local index i, j, the memory S_in entering
// the chunk and chunk-local inclusive cumulative log-gates b:
//   retention  o_i = sum_{j<=i} g^(i-j) (q_i.k_j) v_j + g^(i+1) S_in q_i
//   scalar     o_i = sum_{j<=i} e^(G_i - G_j) (q_i.k_j) v_j + e^(G_i) S_in q_i
//   GLA        o_i = sum_{j<=i} [sum_c q_ic k_jc e^(b_ic - b_jc)] v_j + S_in (q_i . e^(b_i))
// S_in comes from the state pass (bf16 snapshots), so every chunk of every
// sequence is independent: one workgroup per (sequence, chunk) covers all value
// channels and computes the triangle once.
//
// Decomposition (gfx950), NW waves:
//   loads     every global load is issued up front with full-row 16-byte pieces:
//             q, k, v (and the raw gates) for staging, and each wave's slice of
//             S_in, which stays in registers in the A-operand layout;
//   gates     (scalar) one wave scans the chunk's gates into a table of G;
//             (GLA) the raw log-gates are staged and scanned per key channel
//             (16-token runs per lane, joined by shuffles), then folded into bf16
//             operands: q and k rescaled to a reference m_t per 16-token tile and key
//             channel, the cumulative gate r_t just before the tile, moved down to
//             b_last + 80 nats (b_last: at the tile's last token) when the tile's gates
//             sum below -80, so that both factors e^(b - m) and e^(m - b) stay within
//             e^(+-80) for tiles down to -160 (finite in fp32 and bf16); tables
//             F = e^(m_it - m_jt) <= 1 join two tiles in the triangle and R = e^(m_it) <= 1
//             turns rescaled q into q e^(b) for the readout;
//   triangle  the P tiles (it, jt <= it) are spread over the waves; each is one
//             MFMA chain over d_k from LDS, masked and decayed, and stored to LDS
//             in bf16;
//   outputs   wave w owns value pair p = w mod NP (two 16-channel tiles) and every
//             NW/NP-th row tile: the readout S_in q (A = S rows from registers),
//             scaled per token, plus P V with V^T read by ds_read_b64_tr_b16.
#pragma once

#include "chunk_common.hpp"

namespace glr {
namespace ck {

struct OutParams {
    const u16* q;        // [BH][T][DK]
    const u16* k;        // [BH][T][DK]
    const u16* v;        // [BH][T][DV]
    const float* gate;   // retention: log gamma [H]; GLA: log alpha [BH][T][DK]; scalar: log alpha [BH][T]
    const u16* states;   // [BH][NC][DV][DK] memory entering each chunk
    u16* o;              // [BH][T][DV]
    int H, T, NC;
    // GLA's output norm fused in (off when lnw is null): every row of o centred on its mean
    // over the d_v values, divided by sqrt(variance + lneps), times lnw [DV] plus lnb [DV]
    // (lnb may be null)
    const float* lnw;
    const float* lnb;
    float lneps;
};

template <int C, int DK, int DV, int GK>
struct OutLayout {
    static constexpr bool GLA = GK == kGateChannel, SCL = GK == kGateScalar;
    static constexpr int CT = C / 16;
    // bf16 row stride of staged q / k: rows 8 banks apart (d_k + 8 put them 4 apart, and
    // a 16-byte read serves lanes 0-7 with 24-31, rows 0-7 of one piece beside rows 8-15
    // of the next, which then shared a bank in every cycle)
    static constexpr int QS = tile_stride(DK);
    // bf16 row stride of staged v: rows 8 x odd banks apart, so that the 8 rows read
    // by half a wave of ds_read_b64_tr_b16 fall on distinct banks
    static constexpr int VS = DV == 16 ? 16 : DV + 16;
    static constexpr int PS = C + 4;    // bf16 row stride of P
    static constexpr int BS = DK + 4;   // fp32 row stride of the gates
    static constexpr int NF = CT * (CT - 1) / 2;   // off-diagonal tile pairs (GLA table)
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int QB = al(C * QS * 2);
    static constexpr int oQ = 0;                   // q (retention) / q rescaled (GLA)
    static constexpr int oK = oQ + QB;             // k (retention) / k rescaled (GLA)
    static constexpr int oX = oK + QB;
    // region X: v, P and the GLA tables; for GLA it first holds the raw gates
    static constexpr int oV = oX;
    static constexpr int oP = oV + al(C * VS * 2);
    static constexpr int oF = oP + al(C * PS * 2);                  // F = e^(r_it - r_jt), jt < it
    static constexpr int oR = oF + (GLA ? al(NF * DK * 4 + 16) : 0);  // R = e^(r_it)
    static constexpr int oL = oR + (GLA ? al(CT * DK * 4) : 0);    // output-norm row statistics
    static constexpr int NPV = DV >= 32 ? DV / 32 : 1;
    static constexpr int LSTAT = C * NPV * 2;                        // floats: (mean, M2) per row and part
    static constexpr int endX = oL + (GLA ? al(LSTAT * 4) : 0);
    static constexpr int endG = oX + (GLA ? al(C * BS * 4) : 0);
    static constexpr int oS = endX;                                  // scalar: cumulative gates G
    static constexpr int endS = oS + (SCL ? al(C * 4) : 0);
    static constexpr int bytes = endS > endG ? endS : endG;
    static_assert(bytes <= 160 * 1024, "LDS budget of the output pass exceeded");
};

template <int C, int DK, int DV, int GK, int NW>
__global__ __launch_bounds__(64 * NW)
void output_kernel(OutParams p) {
    using Lay = OutLayout<C, DK, DV, GK>;
    constexpr bool GLA = GK == kGateChannel, SCL = GK == kGateScalar;
    constexpr int CT = C / 16, NT = 64 * NW;
    constexpr int KB = (DK + 31) / 32;
    constexpr int QS = Lay::QS, VS = Lay::VS, PS = Lay::PS, BS = Lay::BS;
    constexpr int QP = C * DK / 8, QP_PER = (QP + NT - 1) / NT;    // 16-byte q/k pieces
    constexpr int VP = C * DV / 8, VP_PER = (VP + NT - 1) / NT;    // 16-byte v pieces
    constexpr int GP = GLA ? C * DK / 4 : 0, GP_PER = GLA ? (GP + NT - 1) / NT : 1;
    constexpr int NP = DV >= 32 ? DV / 32 : 1;                    // value pairs (one tile if DV = 16)
    static_assert(NW % NP == 0, "waves must cover the value pairs evenly");
    constexpr int NPAIR = CT * (CT + 1) / 2;

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sQ = reinterpret_cast<u16*>(smem + Lay::oQ);
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    u16* const sV = reinterpret_cast<u16*>(smem + Lay::oV);
    u16* const sP = reinterpret_cast<u16*>(smem + Lay::oP);
    float* const sF = reinterpret_cast<float*>(smem + Lay::oF);
    float* const sR = reinterpret_cast<float*>(smem + Lay::oR);
    float* const sB = reinterpret_cast<float*>(smem + Lay::oX);
    float* const sGs = reinterpret_cast<float*>(smem + Lay::oS);
    float* const sL = reinterpret_cast<float*>(smem + Lay::oL);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;

    const int bh = blockIdx.x / p.NC, c = blockIdx.x % p.NC;
    const int h = bh % p.H;
    const int T = p.T;
    const int t0 = c * C, n = (T - t0 < C) ? (T - t0) : C;
    const int64_t tok0 = static_cast<int64_t>(bh) * T + t0;
    const u16* qc = p.q + tok0 * DK;
    const u16* kc = p.k + tok0 * DK;
    const u16* vc = p.v + tok0 * DV;
    const u16* sc = p.states + (static_cast<int64_t>(bh) * p.NC + c) * DV * DK;
    const float lg2 = (GK == kGateFixed) ? p.gate[h] * kLog2e : 0.f;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};

    // ---- all global loads up front (rows past the end read row 0, zeroed on use)
    u16x8 rq[QP_PER], rk[QP_PER], rv[VP_PER];
    f32x4 rg[GP_PER];
    // scalar gates: wave 0 lane t < n holds token t's
    const float rgs = (SCL && tid < n) ? p.gate[tok0 + tid] : 0.f;
#pragma unroll
    for (int i = 0; i < QP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
        const unsigned off = (idx < QP && j < n) ? static_cast<unsigned>(j * DK + col) : 0u;
        rq[i] = *reinterpret_cast<const u16x8*>(qc + off);
        rk[i] = *reinterpret_cast<const u16x8*>(kc + off);
    }
#pragma unroll
    for (int i = 0; i < VP_PER; ++i) {
        const int idx = tid + i * NT;
        const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
        rv[i] = *reinterpret_cast<const u16x8*>(vc + ((idx < VP && j < n) ? static_cast<unsigned>(j * DV + col) : 0u));
    }
    if constexpr (GLA) {
        const float* gc = p.gate + tok0 * DK;
#pragma unroll
        for (int i = 0; i < GP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DK / 4), col = (idx % (DK / 4)) * 4;
            rg[i] = ldf4(gc + ((idx < GP && j < n) ? static_cast<unsigned>(j * DK + col) : 0u));
        }
    }
    // this wave's rows of S_in in the A-operand layout: tile tt, row m = r16 <-> value
    // channel 32pp + 16tt + m (one 16-row tile when DV = 16)
    const int pp = w % NP;
    u16x8 sa[2][KB];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int vrow = (DV >= 32) ? 32 * pp + 16 * tt + r16 : r16;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            sa[tt][kb] = (col < DK && (DV >= 32 || tt == 0))
                             ? *reinterpret_cast<const u16x8*>(sc + static_cast<unsigned>(vrow * DK + col)) : z8;
        }
    }

    // GLA's output norm: its weight and bias at this wave's channels 32pp + 16tt + 4g + e
    // (the same for every output round), requested with the other global loads
    const bool ln = GLA && p.lnw != nullptr;
    constexpr int NT2 = DV >= 32 ? 2 : 1;
    f32x4 lw[2] = {zf4(), zf4()}, lbv[2] = {zf4(), zf4()};
    if constexpr (GLA) {
        if (ln) {
#pragma unroll
            for (int tt = 0; tt < NT2; ++tt) {
                const int c4 = (DV >= 32 ? 32 * pp + 16 * tt : 0) + 4 * g;
                lw[tt] = ldf4(p.lnw + c4);
                if (p.lnb) lbv[tt] = ldf4(p.lnb + c4);
            }
        }
    }

    auto row_ok = [&](int idx, int per_row, int total) { return idx < total && idx / per_row < n; };

    if constexpr (!GLA) {
        // ---- stage q, k, v
#pragma unroll
        for (int i = 0; i < QP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < QP) {
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                const bool ok = row_ok(idx, DK / 8, QP);
                *reinterpret_cast<u16x8*>(sQ + j * QS + col) = ok ? rq[i] : z8;
                *reinterpret_cast<u16x8*>(sK + j * QS + col) = ok ? rk[i] : z8;
            }
        }
#pragma unroll
        for (int i = 0; i < VP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < VP) {
                const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
                *reinterpret_cast<u16x8*>(sV + j * VS + col) = row_ok(idx, DV / 8, VP) ? rv[i] : z8;
            }
        }
        if constexpr (SCL) {
            // chunk-local inclusive cumulative gates (log2 units; padded tokens add 0)
            if (w == 0) {
                const float G = wave_inclusive_scan(rgs * kLog2e);
                if (lane < C) sGs[lane] = G;
            }
        }
        lds_barrier();
    } else {
        // ---- raw gates (log2 units) -> region X, then a scan per key channel
#pragma unroll
        for (int i = 0; i < GP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < GP) {
                const int j = idx / (DK / 4), col = (idx % (DK / 4)) * 4;
                stf4(sB + j * BS + col, row_ok(idx, DK / 4, GP) ? rg[i] * kLog2e : zf4());
            }
        }
        lds_barrier();
        // chunk-local inclusive cumulative gates: lane (key 16w' + r16, run g) scans
        // tokens 16g .. 16g + 15 of its key channel, runs are joined over g by shuffles
        for (int kt = w; kt < DK / 16; kt += NW) {
            const int key = 16 * kt + r16;
            float t[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) t[e] = (16 * g + e < C) ? sB[(16 * g + e) * BS + key] : 0.f;
#pragma unroll
            for (int e = 1; e < 16; ++e) t[e] += t[e - 1];
            float inc = t[15];
            float y = __shfl_up(inc, 16, 64);
            if (g >= 1) inc += y;
            y = __shfl_up(inc, 32, 64);
            if (g >= 2) inc += y;
            const float base = inc - t[15];
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (16 * g + e < C) sB[(16 * g + e) * BS + key] = t[e] + base;
        }
        lds_barrier();
        // ---- q rescaled to its tile's reference m (the cumulative gate just before the
        // tile, at most 80 nats above the gate at its last token), k rescaled by
        // e^(m - b); the joining table F
#pragma unroll
        for (int i = 0; i < QP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < QP) {
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                const int t = j / 16;
                const bool ok = row_ok(idx, DK / 8, QP);
                const float* bj = sB + j * BS + col;
                const f32x4 b0 = ldf4(bj), b1 = ldf4(bj + 4);
                f32x4 r0 = zf4(), r1 = zf4();
                if (t > 0) {
                    r0 = ldf4(sB + (16 * t - 1) * BS + col);
                    r1 = ldf4(sB + (16 * t - 1) * BS + col + 4);
                }
                r0 = tile_ref4(r0, ldf4(sB + (16 * t + 15) * BS + col));
                r1 = tile_ref4(r1, ldf4(sB + (16 * t + 15) * BS + col + 4));
                float qs[8], ks[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float b = e < 4 ? b0[e] : b1[e - 4];
                    const float r = e < 4 ? r0[e] : r1[e - 4];
                    const float qv = ok ? bf16_bits_to_f32(rq[i][e]) : 0.f;
                    const float kv = ok ? bf16_bits_to_f32(rk[i][e]) : 0.f;
                    qs[e] = qv * ex2(b - r);
                    ks[e] = kv * ex2(r - b);
                }
                *reinterpret_cast<bf16x8*>(sQ + j * QS + col) = pack8(qs[0], qs[1], qs[2], qs[3], qs[4], qs[5], qs[6], qs[7]);
                *reinterpret_cast<bf16x8*>(sK + j * QS + col) = pack8(ks[0], ks[1], ks[2], ks[3], ks[4], ks[5], ks[6], ks[7]);
            }
        }
        // F[(it, jt)][key] = e^(m_it - m_jt), jt < it, pairs in row order; kept in
        // registers until the gates are dead
        constexpr int NFI = Lay::NF * DK, NF_PER = NFI > 0 ? (NFI + NT - 1) / NT : 1;
        float fr[NF_PER];
#pragma unroll
        for (int i = 0; i < NF_PER; ++i) {
            const int idx = tid + i * NT;
            fr[i] = 1.f;
            if (idx < NFI) {
                const int key = idx % DK;
                int pr = idx / DK, it = 1;
                while (pr >= it) { pr -= it; ++it; }   // pair (it, jt = pr), jt < it
                const float ri = tile_ref(sB[(16 * it - 1) * BS + key], sB[(16 * it + 15) * BS + key]);
                const float rj = tile_ref(pr > 0 ? sB[(16 * pr - 1) * BS + key] : 0.f, sB[(16 * pr + 15) * BS + key]);
                fr[i] = ex2(ri - rj);
            }
        }
        // R[it][key] = e^(m_it): the readout operand q e^b is q rescaled times R
        constexpr int NRI = CT * DK, NR_PER = (NRI + NT - 1) / NT;
        float rr[NR_PER];
#pragma unroll
        for (int i = 0; i < NR_PER; ++i) {
            const int idx = tid + i * NT;
            const int it = idx / DK, key = idx % DK;
            rr[i] = idx < NRI ? ex2(tile_ref(it > 0 ? sB[(16 * it - 1) * BS + key] : 0.f, sB[(16 * it + 15) * BS + key]))
                              : 1.f;
        }
        lds_barrier();   // gates dead: region X takes v, P, F and R
#pragma unroll
        for (int i = 0; i < NF_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < NFI) sF[idx] = fr[i];
        }
#pragma unroll
        for (int i = 0; i < NR_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < NRI) sR[idx] = rr[i];
        }
#pragma unroll
        for (int i = 0; i < VP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < VP) {
                const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
                *reinterpret_cast<u16x8*>(sV + j * VS + col) = row_ok(idx, DV / 8, VP) ? rv[i] : z8;
            }
        }
        lds_barrier();
    }

    // ---- triangle: P tiles spread over the waves, pairs (it, jt <= it) in row order
    for (int pr0 = w; pr0 < NPAIR; pr0 += NW) {
        int it = 0, jt = pr0;
        while (jt > it) { jt -= it + 1; ++it; }
        const int i = 16 * it + r16;
        float gi = 0.f;
        f32x4 gj = zf4();
        if constexpr (SCL) {
            gi = sGs[i];
            gj = ldf4(sGs + 16 * jt + 4 * g);
        }
        f32x4 acc = zf4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            // k-slots past d_k (d_k = 16: lanes g = 2, 3) hold zeros; the MFMA itself
            // always runs on the whole wave
            const int col = 32 * kb + 8 * g;
            bf16x8 ka = as_bf16x8(z8), qb = as_bf16x8(z8);
            if (col < DK) {
                ka = *reinterpret_cast<const bf16x8*>(sK + (16 * jt + r16) * QS + col);
                qb = *reinterpret_cast<const bf16x8*>(sQ + i * QS + col);
                if constexpr (GLA) {
                    if (jt < it) {
                        const int f = (it * (it - 1)) / 2 + jt;
                        const f32x4 f0 = ldf4(sF + f * DK + col), f1 = ldf4(sF + f * DK + col + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            qb[e] = static_cast<__bf16>(static_cast<float>(qb[e]) * f0[e]);
                            qb[4 + e] = static_cast<__bf16>(static_cast<float>(qb[4 + e]) * f1[e]);
                        }
                    }
                }
            }
            acc = mfma_16x16x32(ka, qb, acc);
        }
        // acc[r] = P[i][j], i = 16it + r16, j = 16jt + 4g + r
        bf16x4 pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * g + r;
            float val = acc[r];
            if constexpr (GK == kGateFixed) val *= ex2(static_cast<float>(i - j) * lg2);
            if constexpr (SCL) val *= ex2(gi - gj[r]);   // <= 1 for j <= i; the rest is masked
            pv[r] = static_cast<__bf16>((j <= i) ? val : 0.f);
        }
        st4(sP + i * PS + 16 * jt + 4 * g, pv);
    }
    lds_barrier();

    // ---- outputs: readout of S_in plus P V, items (row tile it, value pair pp), in rounds of
    // NW items; the NP items of one row tile fall in one round. With GLA's output norm fused
    // in, every round's rows are kept in registers, each wave writes its rows' partial
    // statistics (mean and sum of squared deviations over its channels) to LDS, and after
    // one barrier every wave normalises and stores its rows
    constexpr int NITEM = CT * NP, ROUNDS = (NITEM + NW - 1) / NW;
    f32x4 keep[GLA ? ROUNDS : 1][2];
    auto store_rows = [&](int i, const f32x4* o2) __attribute__((always_inline)) {
        // lane holds o[i][32pp + 16tt + 4g + r]
        u16* orow = p.o + (tok0 + i) * DV;
        if constexpr (DV >= 32) {
            st4(orow + 32 * pp + 4 * g, cvt4(o2[0]));
            st4(orow + 32 * pp + 16 + 4 * g, cvt4(o2[1]));
        } else {
            st4(orow + 4 * g, cvt4(o2[0]));
        }
    };
#pragma unroll
    for (int round = 0; round < ROUNDS; ++round) {
        const int item = round * NW + w;
        if (!ln && item >= NITEM) break;
        const bool act = item < NITEM;
        const int it = act ? item / NP : 0;
        const int i = 16 * it + r16;
        const float oscale = GLA ? 1.f : SCL ? ex2(sGs[i]) : ex2(static_cast<float>(i + 1) * lg2);
        bf16x8 qb[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int col = 32 * kb + 8 * g;
            qb[kb] = (col < DK) ? *reinterpret_cast<const bf16x8*>(sQ + i * QS + col) : as_bf16x8(z8);
            if constexpr (GLA) {
                // q e^b = (q e^(b - m_it)) e^(m_it)
                if (col < DK) {
                    const f32x4 f0 = ldf4(sR + it * DK + col), f1 = ldf4(sR + it * DK + col + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        qb[kb][e] = static_cast<__bf16>(static_cast<float>(qb[kb][e]) * f0[e]);
                        qb[kb][4 + e] = static_cast<__bf16>(static_cast<float>(qb[kb][4 + e]) * f1[e]);
                    }
                }
            }
        }
        bf16x8 pb[(CT + 1) / 2];
#pragma unroll
        for (int jb = 0; jb < (CT + 1) / 2; ++jb) {
            if (2 * jb <= it) {
                const u16* prow = sP + i * PS + 32 * jb + 4 * g;
                pb[jb] = join8(ld4(prow), (2 * jb + 1 <= it) ? ld4(prow + 16) : zero4());
            }
        }
        f32x4 o2[2];
#pragma unroll
        for (int tt = 0; tt < (DV >= 32 ? 2 : 1); ++tt) {
            f32x4 acc = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc = mfma_16x16x32(as_bf16x8(sa[tt][kb]), qb[kb], acc);
            acc = acc * oscale;
#pragma unroll
            for (int jb = 0; jb < (CT + 1) / 2; ++jb) {
                if (2 * jb <= it) {
                    const bool hi = 2 * jb + 1 <= it;
                    const int c0 = (DV >= 32) ? 32 * pp + 16 * tt : 0;
                    const bf16x8 va = join8(tr_op<VS>(sV, 32 * jb, c0, r16, g),
                                            hi ? tr_op<VS>(sV, 32 * jb + 16, c0, r16, g) : zero4());
                    acc = mfma_16x16x32(va, pb[jb], acc);
                }
            }
            o2[tt] = acc;
        }
        if constexpr (GLA) {
            if (ln) {
                constexpr int CH = 16 * NT2;
                float sum = 0.f;
#pragma unroll
                for (int tt = 0; tt < NT2; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum += o2[tt][e];
                sum += __shfl_xor(sum, 16, 64);
                sum += __shfl_xor(sum, 32, 64);
                const float mp = sum * (1.f / CH);
                float m2 = 0.f;
#pragma unroll
                for (int tt = 0; tt < NT2; ++tt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) m2 += (o2[tt][e] - mp) * (o2[tt][e] - mp);
                m2 += __shfl_xor(m2, 16, 64);
                m2 += __shfl_xor(m2, 32, 64);
                if (act && g == 0) {
                    sL[(i * NP + pp) * 2] = mp;
                    sL[(i * NP + pp) * 2 + 1] = m2;
                }
                keep[round][0] = o2[0];
                keep[round][1] = o2[1];
                continue;
            }
        }
        if (act && i < n) store_rows(i, o2);
    }
    if constexpr (GLA) {
        if (ln) {
            lds_barrier();
#pragma unroll
            for (int round = 0; round < ROUNDS; ++round) {
                const int item = round * NW + w;
                const int i = 16 * (item / NP) + r16;
                if (item < NITEM && i < n) {
                    constexpr int CH = 16 * NT2;
                    float mean = 0.f;
#pragma unroll
                    for (int q2 = 0; q2 < NP; ++q2) mean += sL[(i * NP + q2) * 2];
                    mean *= 1.f / NP;
                    float tot = 0.f;
#pragma unroll
                    for (int q2 = 0; q2 < NP; ++q2) {
                        const float dm = sL[(i * NP + q2) * 2] - mean;
                        tot += sL[(i * NP + q2) * 2 + 1] + CH * dm * dm;
                    }
                    const float rstd = 1.f / sqrtf(tot * (1.f / DV) + p.lneps);
                    f32x4 o2[2];
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) o2[tt] = (keep[round][tt] - mean) * rstd * lw[tt] + lbv[tt];
                    store_rows(i, o2);
                }
            }
        }
    }
}

}  // namespace ck
}  // namespace glr
