// Backward of the chunked forward with a gate per key channel (GLA), bf16 storage.
//
// Method: reverse-mode differentiation of S_t = S_{t-1} Diag(a_t) + v_t k_t^T, o_t = S_t q_t
// ("Scrivere meglio nella memoria", section "Dimenticare: i gate", the diagonal gate),
// organised like the chunkwise forward. With G[j][c] the chunk-local inclusive cumulative
// log-gate of token j and key channel c, S_in the memory entering the chunk and R the
// gradient of the loss with respect to the memory at its last token:
//   dq_i[c] = sum_{j<=i} (do_i . v_j) k_j[c] e^(G_i[c] - G_j[c]) + e^(G_i[c]) (S_in^T do_i)[c]
//   dk_j[c] = sum_{i>=j} (do_i . v_j) q_i[c] e^(G_i[c] - G_j[c]) + e^(G_last[c] - G_j[c]) (R^T v_j)[c]
//   dv_j    = sum_{i>=j} P_ij do_i + R (k_j e^(G_last - G_j)),  P_ij = sum_c q_i[c] k_j[c] e^(G_i[c] - G_j[c])
// and, per key channel (each term of o_t carries e^(B_t[c]) on channel c, each write of token
// j carries e^(-B_j[c])), d log a_t[c] = sum_{s>=t} (q_s[c] dq_s[c] - k_s[c] dk_s[c]) +
// sum_m dS_T[m][c] S_T[m][c].
//
// The decays inside a chunk factor through a reference per 16-token tile, as in the
// forward: r_t[c] = G just before tile t (at most 80 nats above G at its last token),
// q~_i = q_i e^(G_i - r_it), k~_j = k_j e^(r_jt - G_j) (both within e^(+-80) for tiles whose
// gates sum to -160 or more), F_(it,jt) = e^(r_it - r_jt) <= 1, so
// e^(G_i - G_j) = q~-scale * F * k~-scale on every product:
//   P = (Q~ . F) K~^T per tile pair;  dK^T = e^(r_jt - G_j) . (Q~ . F)^T A2 + e^(G_last - G_j) . R^T V^T
//   dQ^T = e^(G_i - r_it) . (K~ . F)^T A2^T + e^(G_i) . S_in^T dO^T;  dV^T = dO^T P + R K^^T,
// K^ = K~ e^(G_last - r_jt), A2 = dO V^T masked (no decay), the F factors applied to the
// operand rows (one per lane per 16-token half), the element factors to the results.
//
// The gate gradient needs no pass of its own: summed over the tokens after chunk c it is
// the per-channel d log a of chunk c + 1's first token, sum_m R_c[m][c] S_out[m][c] (the
// gradient at chunk c's end against the memory there: S_in of chunk c + 1, or S_T), so each
// chunk writes d log a_t[c] = (sum over its tokens s >= t of q_s[c] dq_s[c] - k_s[c] dk_s[c])
// + sum_m R_c[m][c] S_out[m][c] directly.
//
// Gradient pass (gfx950): persistent workgroups of eight waves, one per CU, each taking
// (sequence, chunk) items in turn. An item loads q, k, v, dO, its gates and R as it starts,
// S_in and S_out while its tables are built (holding the next item's operands in registers
// during the products needs more than the 256 registers two waves per SIMD leave, and
// the spills cost more than the wait). Tiles in LDS use
// the chunk-swizzled layout; the cumulative gates are an fp32 [C][d_k + 4] table. A wave
// that computes the dK tile of (feature tile, token tile) also computes the dQ tile of the
// same pair, so q . dq - k . dk per element is formed in registers; the chunk's reverse
// scan of it per channel runs in LDS after the products.
#pragma once

#include "chunk_backward.hpp"

namespace glr {
namespace ck {

struct GradGlaParams {
    const u16* q;          // [BH][T][DK]
    const u16* k;          // [BH][T][DK]
    const u16* v;          // [BH][T][DV]
    const u16* dout;       // [BH][T][DV]
    const float* gate;     // log alpha [BH][T][DK]
    const u16* s_in;       // [BH][NC][DV][DK] forward snapshots
    const u16* r;          // [BH][NC][DV][DK] backward snapshots
    u16* dq;               // [BH][T][DK]
    u16* dk;               // [BH][T][DK]
    u16* dv;               // [BH][T][DV]
    const float* s_fin;    // [BH][DV][DK] fp32 final memory (S_out of the last chunk)
    float* dgate;          // [BH][T][DK] gradient of log alpha
    int T, NC, items;
};

template <int C, int DK, int DV>
struct GradGlaLayout {
    using TQ = SwzTile<DK>;
    using TV = SwzTile<DV>;
    using TA = SwzTile<C>;
    static constexpr int CT = C / 16;
    static constexpr int NF = CT * (CT - 1) / 2;   // tile pairs jt < it
    static constexpr int GS = DK + 4;              // fp32 row stride of the gate table
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int oQ = 0;                                         // q~
    static constexpr int oK = oQ + al(C * TQ::STRIDE * 2);               // k~
    static constexpr int oV = oK + al(C * TQ::STRIDE * 2);
    static constexpr int oO = oV + al(C * TV::STRIDE * 2);
    static constexpr int oA1 = oO + al(C * TV::STRIDE * 2);              // P
    static constexpr int oA2 = oA1 + al(C * TA::STRIDE * 2);
    static constexpr int oX = oA2 + al(C * TA::STRIDE * 2);              // R, then S_in
    static constexpr int oG = oX + al(DV * TQ::STRIDE * 2);              // G [C][GS] (log2 units)
    static constexpr int oF = oG + al(C * GS * 4);                       // F [NF][DK]
    static constexpr int oL = oF + al((NF > 0 ? NF : 1) * DK * 4);       // e^(G_last - r_t) [CT][DK]
    static constexpr int oR = oL + al(CT * DK * 4);                      // r_t [CT][DK] (log2)
    static constexpr int oO2 = oR + al(CT * DK * 4);                     // per-wave offsets [8][DK]
    static constexpr int bytes = oO2 + al(8 * DK * 4);
    static_assert(bytes <= 160 * 1024, "LDS budget of the GLA gradient pass exceeded");
};

// pair index of tile pair (it, jt), jt < it, in row order
__device__ __forceinline__ int gla_pair(int it, int jt) { return it * (it - 1) / 2 + jt; }

template <int C, int DK, int DV>
__global__ __launch_bounds__(512)
void grad_gla_kernel(GradGlaParams p) {
    using Lay = GradGlaLayout<C, DK, DV>;
    using TQ = typename Lay::TQ;
    using TV = typename Lay::TV;
    using TA = typename Lay::TA;
    constexpr int NT = 512, NW = 8;
    constexpr int CT = C / 16, JB = (CT + 1) / 2, GS = Lay::GS;
    constexpr int KB = (DK + 31) / 32, VB = (DV + 31) / 32;
    constexpr int QP = C * DK / 8, QP_PER = (QP + NT - 1) / NT;
    constexpr int VP = C * DV / 8, VP_PER = (VP + NT - 1) / NT;
    constexpr int XP = DV * DK / 8, XP_PER = (XP + NT - 1) / NT;
    constexpr int GP = C * DK / 4, GP_PER = (GP + NT - 1) / NT;
    constexpr int FK = DK / 16, FV = DV / 16;
    constexpr int MAXT = (FK * CT + NW - 1) / NW;   // dK (and dQ) tiles per wave

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sQ = reinterpret_cast<u16*>(smem + Lay::oQ);
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    u16* const sV = reinterpret_cast<u16*>(smem + Lay::oV);
    u16* const sO = reinterpret_cast<u16*>(smem + Lay::oO);
    u16* const sA1 = reinterpret_cast<u16*>(smem + Lay::oA1);
    u16* const sA2 = reinterpret_cast<u16*>(smem + Lay::oA2);
    u16* const sX = reinterpret_cast<u16*>(smem + Lay::oX);
    float* const sG = reinterpret_cast<float*>(smem + Lay::oG);
    float* const sF = reinterpret_cast<float*>(smem + Lay::oF);
    float* const sL = reinterpret_cast<float*>(smem + Lay::oL);
    float* const sR = reinterpret_cast<float*>(smem + Lay::oR);
    float* const sOff = reinterpret_cast<float*>(smem + Lay::oO2);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int T = p.T;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};

    // ---- operands of an item in registers (rows past the end read row 0, zeroed on use):
    // q, k, v, dO, R and the gates when the item starts, S_in and S_out after its staging
    u16x8 rq[QP_PER], rk[QP_PER], rv[VP_PER], ro[VP_PER], rx[XP_PER], rs[XP_PER], rn[XP_PER];
    f32x4 rg[GP_PER];
    auto load_item = [&](int item) {
        const int lbh = item / p.NC, lc = item % p.NC;
        const int lt0 = lc * C, ln = (T - lt0 < C) ? (T - lt0) : C;
        const int64_t ltok0 = static_cast<int64_t>(lbh) * T + lt0;
#pragma unroll
        for (int i = 0; i < QP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
            const unsigned off = (idx < QP && j < ln) ? static_cast<unsigned>(j * DK + col) : 0u;
            rq[i] = *reinterpret_cast<const u16x8*>(p.q + ltok0 * DK + off);
            rk[i] = *reinterpret_cast<const u16x8*>(p.k + ltok0 * DK + off);
        }
#pragma unroll
        for (int i = 0; i < VP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            const unsigned off = (idx < VP && j < ln) ? static_cast<unsigned>(j * DV + col) : 0u;
            rv[i] = *reinterpret_cast<const u16x8*>(p.v + ltok0 * DV + off);
            ro[i] = *reinterpret_cast<const u16x8*>(p.dout + ltok0 * DV + off);
        }
    };
    // R and the gates of the current item, loaded when the item starts
    auto load_rg = [&](int item) {
        const int lbh = item / p.NC, lc = item % p.NC;
        const int lt0 = lc * C, ln = (T - lt0 < C) ? (T - lt0) : C;
        const int64_t ltok0 = static_cast<int64_t>(lbh) * T + lt0;
        const int64_t lchunk = static_cast<int64_t>(lbh) * p.NC + lc;
#pragma unroll
        for (int i = 0; i < XP_PER; ++i) {
            const int idx = tid + i * NT;
            const unsigned off = (idx < XP) ? static_cast<unsigned>(idx * 8) : 0u;
            rx[i] = *reinterpret_cast<const u16x8*>(p.r + lchunk * DV * DK + off);
        }
#pragma unroll
        for (int i = 0; i < GP_PER; ++i) {
            const int idx = tid + i * NT;
            const int j = idx / (DK / 4), col = (idx % (DK / 4)) * 4;
            const unsigned off = (idx < GP && j < ln) ? static_cast<unsigned>(j * DK + col) : 0u;
            rg[i] = ldf4(p.gate + ltok0 * DK + off);
        }
    };

    // the memories of the current item: S_in, and S_out (the next chunk's S_in, or the final
    // memory in fp32, rounded like the snapshots); loaded at the start of the item, used at
    // the end of its dK phase
    auto load_mem = [&](int item) {
        const int lbh = item / p.NC, lc = item % p.NC;
        const int64_t lchunk = static_cast<int64_t>(lbh) * p.NC + lc;
#pragma unroll
        for (int i = 0; i < XP_PER; ++i) {
            const int idx = tid + i * NT;
            const unsigned off = (idx < XP) ? static_cast<unsigned>(idx * 8) : 0u;
            rs[i] = *reinterpret_cast<const u16x8*>(p.s_in + lchunk * DV * DK + off);
            if (lc + 1 < p.NC) {
                rn[i] = *reinterpret_cast<const u16x8*>(p.s_in + (lchunk + 1) * DV * DK + off);
            } else {
                const float* sf = p.s_fin + static_cast<int64_t>(lbh) * DV * DK + off;
                const f32x4 a0 = ldf4(sf), a1 = ldf4(sf + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rn[i][e] = f32_to_bf16_bits(a0[e]);
                    rn[i][4 + e] = f32_to_bf16_bits(a1[e]);
                }
            }
        }
    };

    int item = blockIdx.x;
    if (item >= p.items) return;
    for (;;) {
        const int bh = item / p.NC, c = item % p.NC;
        const int t0 = c * C, n = (T - t0 < C) ? (T - t0) : C;
        const int64_t tok0 = static_cast<int64_t>(bh) * T + t0;
        load_item(item);
        load_rg(item);

        // ---- stage v, dO, R and the raw gates (log2 units; rows past the end zero)
#pragma unroll
        for (int i = 0; i < VP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < VP) {
                const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
                *reinterpret_cast<u16x8*>(sV + TV::off(j, col)) = (j < n) ? rv[i] : z8;
                *reinterpret_cast<u16x8*>(sO + TV::off(j, col)) = (j < n) ? ro[i] : z8;
            }
        }
        auto stage_x = [&](const u16x8* src) {
#pragma unroll
            for (int i = 0; i < XP_PER; ++i) {
                const int idx = tid + i * NT;
                if (idx < XP) {
                    const int m = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                    *reinterpret_cast<u16x8*>(sX + TQ::off(m, col)) = src[i];
                }
            }
        };
        stage_x(rx);
#pragma unroll
        for (int i = 0; i < GP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < GP) {
                const int j = idx / (DK / 4), col = (idx % (DK / 4)) * 4;
                stf4(sG + j * GS + col, (j < n) ? rg[i] * kLog2e : zf4());
            }
        }
        load_mem(item);   // in flight while the tables and the products of the first half run
        lds_barrier();
        // chunk-local inclusive cumulative gates: lane (key 16kt + r16, run g) scans tokens
        // 16g .. 16g + 15 of its key channel; runs are joined over g by shuffles
        for (int kt = w; kt < DK / 16; kt += NW) {
            const int key = 16 * kt + r16;
            float tv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) tv[e] = (16 * g + e < C) ? sG[(16 * g + e) * GS + key] : 0.f;
#pragma unroll
            for (int e = 1; e < 16; ++e) tv[e] += tv[e - 1];
            float inc = tv[15];
            float y = __shfl_up(inc, 16, 64);
            if (g >= 1) inc += y;
            y = __shfl_up(inc, 32, 64);
            if (g >= 2) inc += y;
            const float base = inc - tv[15];
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (16 * g + e < C) sG[(16 * g + e) * GS + key] = tv[e] + base;
        }
        lds_barrier();

        // ---- tables (references r_t, F, e^(G_last - r_t)) and the rescaled q~, k~
        for (int idx = tid; idx < CT * DK; idx += NT) {
            const int t = idx / DK, key = idx % DK;
            const float rt = tile_ref(t > 0 ? sG[(16 * t - 1) * GS + key] : 0.f, sG[(16 * t + 15) * GS + key]);
            sR[idx] = rt;
            sL[idx] = ex2(sG[(C - 1) * GS + key] - rt);
        }
        for (int idx = tid; idx < Lay::NF * DK; idx += NT) {
            const int key = idx % DK;
            int pr = idx / DK, it = 1;
            while (pr >= it) { pr -= it; ++it; }   // pair (it, jt = pr), jt < it
            const float ri = tile_ref(sG[(16 * it - 1) * GS + key], sG[(16 * it + 15) * GS + key]);
            const float rj = tile_ref(pr > 0 ? sG[(16 * pr - 1) * GS + key] : 0.f, sG[(16 * pr + 15) * GS + key]);
            sF[idx] = ex2(ri - rj);
        }
#pragma unroll
        for (int i = 0; i < QP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < QP) {
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                const int t = j / 16;
                const float* gj = sG + j * GS + col;
                const f32x4 b0 = ldf4(gj), b1 = ldf4(gj + 4);
                f32x4 c0 = zf4(), c1 = zf4();
                if (t > 0) {
                    c0 = ldf4(sG + (16 * t - 1) * GS + col);
                    c1 = ldf4(sG + (16 * t - 1) * GS + col + 4);
                }
                c0 = tile_ref4(c0, ldf4(sG + (16 * t + 15) * GS + col));
                c1 = tile_ref4(c1, ldf4(sG + (16 * t + 15) * GS + col + 4));
                float qs[8], ks[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float b = e < 4 ? b0[e] : b1[e - 4];
                    const float r = e < 4 ? c0[e] : c1[e - 4];
                    const float qv = (j < n) ? bf16_bits_to_f32(rq[i][e]) : 0.f;
                    const float kv = (j < n) ? bf16_bits_to_f32(rk[i][e]) : 0.f;
                    qs[e] = qv * ex2(b - r);
                    ks[e] = kv * ex2(r - b);
                }
                *reinterpret_cast<bf16x8*>(sQ + TQ::off(j, col)) = pack8(qs[0], qs[1], qs[2], qs[3], qs[4], qs[5], qs[6], qs[7]);
                *reinterpret_cast<bf16x8*>(sK + TQ::off(j, col)) = pack8(ks[0], ks[1], ks[2], ks[3], ks[4], ks[5], ks[6], ks[7]);
            }
        }
        const int step = static_cast<int>(gridDim.x);
        const int next = (item < p.items - step) ? item + step : p.items;
        lds_barrier();

        // F factor of tile pair (it, jt) for key channel `key`: 1 on the diagonal and above
        // (above, the products it multiplies are masked to zero)
        auto fac = [&](int it, int jt, int key) { return jt < it ? sF[gla_pair(it, jt) * DK + key] : 1.f; };

        // ---- P = (Q~ . F) K~^T and A2 = dO V^T, every tile (upper ones zero):
        // acc[r] = X[i = 16it + r16][j = 16jt + 4g + r]
        for (int t = w; t < 2 * CT * CT; t += NW) {
            const bool second = t >= CT * CT;
            const int it = (t % (CT * CT)) / CT, jt = t % CT;
            const int i = 16 * it + r16;
            u16* const dst = second ? sA2 : sA1;
            bf16x4 pv = zero4();
            if (jt <= it) {
                f32x4 acc = zf4();
                const int ar = 16 * jt + r16;
                const int D = second ? DV : DK;
#pragma unroll
                for (int kb = 0; kb < (KB > VB ? KB : VB); ++kb) {
                    const int col = rr_col(kb, g, KB > VB ? KB : VB);
                    bf16x8 a8 = as_bf16x8(z8), b8 = as_bf16x8(z8);
                    if (col < D) {
                        a8 = *reinterpret_cast<const bf16x8*>(second ? sV + TV::off(ar, col) : sK + TQ::off(ar, col));
                        b8 = *reinterpret_cast<const bf16x8*>(second ? sO + TV::off(i, col) : sQ + TQ::off(i, col));
                        if (!second && jt < it) {
                            const float* f = sF + gla_pair(it, jt) * DK + col;
                            const f32x4 f0 = ldf4(f), f1 = ldf4(f + 4);
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                b8[e] = static_cast<__bf16>(static_cast<float>(b8[e]) * f0[e]);
                                b8[4 + e] = static_cast<__bf16>(static_cast<float>(b8[4 + e]) * f1[e]);
                            }
                        }
                    }
                    acc = mfma_16x16x32(a8, b8, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jt + 4 * g + r;
                    pv[r] = static_cast<__bf16>((j <= i) ? acc[r] : 0.f);
                }
            }
            st4(dst + TA::off(i, 16 * jt + 4 * g), pv);
        }
        lds_barrier();

        // ---- dV^T tiles (feature tile ft, token tile jt); lane holds D[f = 16ft + 4g + r][j = 16jt + r16]
        for (int t = w; t < FV * CT; t += NW) {
            const int ft = t / CT, jt = t % CT;
            const int j = 16 * jt + r16;
            f32x4 acc = zf4();
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                if (32 * b + 31 < 16 * jt) continue;                 // rows i all above j
                const bool hi = 2 * b + 1 < CT;
                acc = mfma_16x16x32(tr_split_s<DV>(sO, b, 16 * ft, hi, r16, g), tr_split_s<C>(sA1, b, 16 * jt, hi, r16, g),
                                    acc);
            }
            // sum over keys m of R[f][m] K^[j][m], K^ = K~ e^(G_last - r_jt)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int col = rr_col(kb, g, KB);
                bf16x8 xa = as_bf16x8(z8), kb8 = as_bf16x8(z8);
                if (col < DK) {
                    xa = *reinterpret_cast<const bf16x8*>(sX + TQ::off(16 * ft + r16, col));
                    kb8 = *reinterpret_cast<const bf16x8*>(sK + TQ::off(j, col));
                    const f32x4 l0 = ldf4(sL + jt * DK + col), l1 = ldf4(sL + jt * DK + col + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kb8[e] = static_cast<__bf16>(static_cast<float>(kb8[e]) * l0[e]);
                        kb8[4 + e] = static_cast<__bf16>(static_cast<float>(kb8[4 + e]) * l1[e]);
                    }
                }
                acc = mfma_16x16x32(xa, kb8, acc);
            }
            if (j < n) st4(p.dv + (tok0 + j) * DV + 16 * ft + 4 * g, cvt4(acc));
        }

        // ---- dK^T tiles (key tile ft, token tile jt); lane holds D[c = 16ft + 4g + r][j = 16jt + r16].
        // The lane keeps k_j[c] dk_j[c] for the dQ tile of the same pair (same wave, same lane).
        f32x4 gk[MAXT];
#pragma unroll
        for (int s = 0; s < MAXT; ++s) {
            __builtin_amdgcn_sched_barrier(0);   // one tile at a time: bounds the registers in flight
            gk[s] = zf4();
            const int u = w + NW * s;
            if (u >= FK * CT) continue;
            const int ft = u / CT, jt = u % CT;
            const int j = 16 * jt + r16;
            const int cf = 16 * ft + r16;   // the lane's operand row (feature) for the F factors
            f32x4 acc = zf4(), acc2 = zf4();
            // term 1: (Q~ . F)^T A2, rows i of tiles 2b, 2b + 1
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                if (32 * b + 31 < 16 * jt) continue;
                const bool hi = 2 * b + 1 < CT;
                bf16x4 lo4 = tr_op_s<DK>(sQ, 32 * b, 16 * ft, r16, g);
                bf16x4 hi4 = hi ? tr_op_s<DK>(sQ, 32 * b + 16, 16 * ft, r16, g) : zero4();
                const float f0 = fac(2 * b, jt, cf), f1 = hi ? fac(2 * b + 1, jt, cf) : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo4[e] = static_cast<__bf16>(static_cast<float>(lo4[e]) * f0);
                    hi4[e] = static_cast<__bf16>(static_cast<float>(hi4[e]) * f1);
                }
                acc = mfma_16x16x32(join8(lo4, hi4), tr_split_s<C>(sA2, b, 16 * jt, hi, r16, g), acc);
            }
            // term 2: R^T V^T (R read transposed)
#pragma unroll
            for (int b = 0; b < VB; ++b) {
                const bool hi = 32 * b + 16 < DV;
                const int vc = 32 * b + 4 * g;
                const bf16x8 vb = join8(ld4(sV + TV::off(j, vc)), hi ? ld4(sV + TV::off(j, vc + 16)) : zero4());
                acc2 = mfma_16x16x32(tr_split_s<DK>(sX, b, 16 * ft, hi, r16, g), vb, acc2);
            }
            // element factors: term 1 e^(r_jt - G_j), term 2 e^(G_last - G_j)
            const int c4 = 16 * ft + 4 * g;
            const f32x4 gj = ldf4(sG + j * GS + c4), rj = ldf4(sR + jt * DK + c4), gl = ldf4(sG + (C - 1) * GS + c4);
            f32x4 dkv;
#pragma unroll
            for (int r = 0; r < 4; ++r) dkv[r] = acc[r] * ex2(rj[r] - gj[r]) + acc2[r] * ex2(gl[r] - gj[r]);
            if (j < n) {
                st4(p.dk + (tok0 + j) * DK + c4, cvt4(dkv));
                const f32x4 kj = up4(ld4(p.k + (tok0 + j) * DK + c4));
                gk[s] = kj * dkv;
            }
        }
        // chunk offset of the gate gradient, sum_m R[m][c] S_out[m][c], R read back from LDS: a
        // thread's pieces share one group of 8 channels (idx % (DK / 8) does not depend on i);
        // partial sums meet over the wave's lanes of that group, then over the waves in LDS
        {
            float po[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) po[e] = 0.f;
#pragma unroll
            for (int i = 0; i < XP_PER; ++i) {
                const int idx = tid + i * NT;
                if (XP % NT == 0 || idx < XP) {
                    const int m = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                    const u16x8 rr = *reinterpret_cast<const u16x8*>(sX + TQ::off(m, col));
#pragma unroll
                    for (int e = 0; e < 8; ++e) po[e] += bf16_bits_to_f32(rr[e]) * bf16_bits_to_f32(rn[i][e]);
                }
            }
            constexpr int G8 = DK / 8;   // channel groups; lanes l and l + G8 share one
#pragma unroll
            for (int e = 0; e < 8; ++e) {
#pragma unroll
                for (int off = G8; off < 64; off <<= 1) po[e] += __shfl_xor(po[e], off, 64);
            }
            if (lane < G8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) sOff[w * DK + lane * 8 + e] = po[e];
            }
        }
        lds_barrier();   // R is dead: the region takes S_in
        stage_x(rs);
        lds_barrier();

        // ---- dQ^T tiles (key tile ft, token tile it), the same pairs as the dK tiles of this
        // wave; lane holds dQ[i = 16it + r16][c = 16ft + 4g + r]
        f32x4 gqv[MAXT];
#pragma unroll
        for (int s = 0; s < MAXT; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            gqv[s] = zf4();
            const int u = w + NW * s;
            if (u >= FK * CT) continue;
            const int ft = u / CT, it = u % CT;
            const int i = 16 * it + r16;
            const int cf = 16 * ft + r16;
            f32x4 acc = zf4(), acc2 = zf4();
            // term 1: (K~ . F)^T A2^T, rows j of tiles 2b, 2b + 1
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                if (32 * b > 16 * it + 15) continue;                 // columns j all past i
                const bool hi = 2 * b + 1 < CT;
                bf16x4 lo4 = tr_op_s<DK>(sK, 32 * b, 16 * ft, r16, g);
                bf16x4 hi4 = hi ? tr_op_s<DK>(sK, 32 * b + 16, 16 * ft, r16, g) : zero4();
                const float f0 = fac(it, 2 * b, cf), f1 = hi ? fac(it, 2 * b + 1, cf) : 1.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo4[e] = static_cast<__bf16>(static_cast<float>(lo4[e]) * f0);
                    hi4[e] = static_cast<__bf16>(static_cast<float>(hi4[e]) * f1);
                }
                const int ac = 32 * b + 4 * g;
                acc = mfma_16x16x32(join8(lo4, hi4),
                                    join8(ld4(sA2 + TA::off(i, ac)), hi ? ld4(sA2 + TA::off(i, ac + 16)) : zero4()), acc);
            }
            // term 2: S_in^T dO^T
#pragma unroll
            for (int b = 0; b < VB; ++b) {
                const bool hi = 32 * b + 16 < DV;
                const int oc = 32 * b + 4 * g;
                acc2 = mfma_16x16x32(tr_split_s<DK>(sX, b, 16 * ft, hi, r16, g),
                                     join8(ld4(sO + TV::off(i, oc)), hi ? ld4(sO + TV::off(i, oc + 16)) : zero4()), acc2);
            }
            // element factors: term 1 e^(G_i - r_it), term 2 e^(G_i)
            const int c4 = 16 * ft + 4 * g;
            const f32x4 gi = ldf4(sG + i * GS + c4), ri = ldf4(sR + it * DK + c4);
            f32x4 dqv;
#pragma unroll
            for (int r = 0; r < 4; ++r) dqv[r] = acc[r] * ex2(gi[r] - ri[r]) + acc2[r] * ex2(gi[r]);
            if (i < n) {
                st4(p.dq + (tok0 + i) * DK + c4, cvt4(dqv));
                const f32x4 qv = up4(ld4(p.q + (tok0 + i) * DK + c4));
                gqv[s] = qv * dqv - gk[s];
            }
        }
        lds_barrier();   // the gate table is free: it takes q . dq - k . dk per element
#pragma unroll
        for (int s = 0; s < MAXT; ++s) {
            const int u = w + NW * s;
            if (u >= FK * CT) continue;
            const int ft = u / CT, it = u % CT;
            stf4(sG + (16 * it + r16) * GS + 16 * ft + 4 * g, gqv[s]);
        }
        lds_barrier();
        // ---- gate gradients: per key channel, the reverse cumulative sum over the chunk's
        // tokens plus the chunk offset; lane (key 16kt + r16, run g) takes tokens 16g .. 16g + 15
        for (int kt = w; kt < DK / 16; kt += NW) {
            const int key = 16 * kt + r16;
            float off = 0.f;
#pragma unroll
            for (int u = 0; u < NW; ++u) off += sOff[u * DK + key];
            float tv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) tv[e] = (16 * g + e < C) ? sG[(16 * g + e) * GS + key] : 0.f;
#pragma unroll
            for (int e = 14; e >= 0; --e) tv[e] += tv[e + 1];
            // sum of the later runs of this channel
            float inc = tv[0];
            float y = __shfl_down(inc, 16, 64);
            if (g <= 2) inc += y;
            y = __shfl_down(inc, 32, 64);
            if (g <= 1) inc += y;
            const float base = inc - tv[0] + off;
            float* dst = p.dgate + tok0 * DK + key;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (16 * g + e < n) dst[static_cast<int64_t>(16 * g + e) * DK] = tv[e] + base;
        }
        lds_barrier();   // every read of this item's tiles is done before the next staging
        if (next >= p.items) break;
        item = next;
    }
}

// Workspace of a GLA backward call: the forward and the backward snapshots
// ([BH][NC][DV][DK] bf16 each) and the final memory [BH][DV][DK] fp32, each from a
// 256-byte boundary.
inline size_t bwd_gla_workspace_bytes(int64_t heads, int T, int chunk, int dk, int dv) {
    const int64_t nc = (T + chunk - 1) / chunk;
    return 2 * bwd_align(heads * nc * dv * dk * 2) + bwd_align(heads * dv * dk * 4);
}

template <int C, int DK, int DV>
hipError_t launch_backward_gla_dv(const BwdArgs& a, hipStream_t stream) {
    const int NC = (a.T + C - 1) / C;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    unsigned char* base = static_cast<unsigned char*>(a.ws);
    u16* fwd = reinterpret_cast<u16*>(base);
    u16* rev = reinterpret_cast<u16*>(base + bwd_align(heads * NC * DV * DK * 2));
    float* sfin = reinterpret_cast<float*>(base + 2 * bwd_align(heads * NC * DV * DK * 2));
    // forward state pass (snapshots and final memory), then the same walk backwards on (q, dO)
    ChunkArgs f{a.q, a.k, a.v, a.gate, nullptr, a.s0, nullptr, sfin, a.B, a.H, a.T, DK, DV, C, fwd};
    ChunkArgs r{a.q, a.q, a.dout, a.gate, nullptr, a.ds_out, nullptr, a.ds0, a.B, a.H, a.T, DK, DV, C, rev};
    hipError_t err = hipErrorInvalidValue;
    switch (state_value_tiles(heads, DV, DK)) {
        case 8:
            if constexpr (DV >= 128) {
                err = launch_state<C, DK, 8, kGateChannel>(f, NC, stream);
                if (err == hipSuccess) err = launch_state<C, DK, 8, kGateChannel, true>(r, NC, stream);
            }
            break;
        case 4:
            if constexpr (DV >= 64) {
                err = launch_state<C, DK, 4, kGateChannel>(f, NC, stream);
                if (err == hipSuccess) err = launch_state<C, DK, 4, kGateChannel, true>(r, NC, stream);
            }
            break;
        case 2:
            if constexpr (DV >= 32) {
                err = launch_state<C, DK, 2, kGateChannel>(f, NC, stream);
                if (err == hipSuccess) err = launch_state<C, DK, 2, kGateChannel, true>(r, NC, stream);
            }
            break;
        default:
            err = launch_state<C, DK, 1, kGateChannel>(f, NC, stream);
            if (err == hipSuccess) err = launch_state<C, DK, 1, kGateChannel, true>(r, NC, stream);
            break;
    }
    if (err != hipSuccess) return err;
    if (NC == 0) return hipSuccess;
    GradGlaParams p{};
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.dout = static_cast<const u16*>(a.dout);
    p.gate = a.gate;
    p.s_in = fwd;
    p.r = rev;
    p.dq = static_cast<u16*>(a.grad_q);
    p.dk = static_cast<u16*>(a.grad_k);
    p.dv = static_cast<u16*>(a.grad_v);
    p.s_fin = sfin;
    p.dgate = a.dgate;
    p.T = a.T;
    p.NC = NC;
    p.items = static_cast<int>(heads * NC);
    int dev = 0, cus = 256, per_cu = 1;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, grad_gla_kernel<C, DK, DV>, 512, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const int64_t slots = static_cast<int64_t>(cus) * per_cu;
    const int grid = p.items < slots ? p.items : static_cast<int>(slots);
    hipLaunchKernelGGL((grad_gla_kernel<C, DK, DV>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <int C, int DK>
hipError_t launch_backward_gla_dk(const BwdArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_backward_gla_dv<C, DK, 16>(a, stream);
        case 32: return launch_backward_gla_dv<C, DK, 32>(a, stream);
        case 64: return launch_backward_gla_dv<C, DK, 64>(a, stream);
        case 128: return launch_backward_gla_dv<C, DK, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int C>
hipError_t launch_backward_gla(const BwdArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_backward_gla_dk<C, 16>(a, stream);
        case 32: return launch_backward_gla_dk<C, 32>(a, stream);
        case 64: return launch_backward_gla_dk<C, 64>(a, stream);
        case 128: return launch_backward_gla_dk<C, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
