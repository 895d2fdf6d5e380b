// State pass of the two-pass chunked forward for retention, the scalar
// data-dependent decay and GLA (bf16 storage).
//
// Method: the chunkwise form of retention ("Le architetture lineari: RetNet,
// RWKV, xLSTM", section "RetNet: la retention e le sue tre forme", Fig. 16.5)
// and its per-channel gated extension ("Scrivere meglio nella memoria",
// section "Dimenticare: i gate", diagonal-gate equation). Only the memory
// passes from one chunk to the next; with chunk-local inclusive cumulative
// log-gates b_j (per key channel) and n tokens in the chunk:
//   retention  S_out = g^n S_in + sum_j g^(n-1-j) v_j k_j^T
//   scalar     S_out = e^(G_{n-1}) S_in + sum_j e^(G_{n-1} - G_j) v_j k_j^T (G: the
//              chunk-local inclusive cumulative log of one gate per token)
//   GLA        S_out = S_in Diag(e^(b_{n-1})) + sum_j v_j (k_j . e^(b_{n-1} - b_j))^T
// This kernel walks the chunks of one sequence in order and writes, for every
// chunk c, the memory entering it (bf16, [d_v][d_k]) to a workspace; the output
// pass then evaluates all chunks in parallel from those snapshots.
//
// REV (the backward): the same walk from the last chunk to the first carries the
// gradient R of the loss with respect to the memory at a chunk's last token,
// R_(c-1) = R_c Diag(e^(G_last)) + sum_i dO_i (q_i e^(G_i))^T - the forward carry with
// q in place of k, dO in place of v and the weights e^(G_j) (per key channel for
// GLA) in place of e^(G_last - G_j); the snapshot of chunk c is R_c, and what is left
// after chunk 0 is the gradient of S_0.
//
// Decomposition (gfx950). Transitions act on key channels (columns of S) and
// the write is an outer product, so every element of S evolves on its own. A
// workgroup owns a DKB x DVB block (DKB = 16 NW key channels, DVB = 16 TV value
// channels); each of its NWK x NWV waves keeps one key tile against every NWV-th
// value tile in fp32 MFMA accumulators for the whole sequence. Keys, values (and raw gates) are staged
// per workgroup with full-row 16-byte loads - narrower per-wave tiles would
// multiply the memory requests per CU, which bound this pass. Chunks go in
// groups of U per workgroup barrier:
//   carry     per chunk of the group, the weighted key operand (carry factor
//             applied in registers to the ds_read_b64_tr_b16 result) and V^T give
//             the chunk's own contribution dS on MFMA, into separate accumulators,
//             so the U products overlap; then, in order, the entering memory is
//             stored (bf16) and S <- decay . S + dS;
//   gates     (scalar) a wave prefix scan over the chunk's tokens, the lane's
//             weights fetched by shuffles;
//             (GLA) each lane reads the raw log-gates of its key channel for the
//             tokens it holds in the operand layout, scans its 4-token runs and
//             joins runs across the four lanes of the channel with shuffles;
//   staging   the next group goes from registers to the other LDS buffer;
//   prefetch  HBM loads run ahead through a two-slot register ring of groups.
#pragma once

#include <type_traits>

#include "chunk_common.hpp"

namespace glr {
namespace ck {

struct StateParams {
    const u16* k;        // [BH][T][DK]
    const u16* v;        // [BH][T][dv]
    const float* gate;   // retention: log gamma [H]; GLA: log alpha [BH][T][DK]; scalar: log alpha [BH][T]
    const float* s0;     // [BH][dv][DK] or null
    u16* states;         // [BH][NC][dv][DK]: memory entering each chunk
    float* s_out;        // [BH][dv][DK] or null
    int H, T, dv, NC, vblocks, kblocks, remap;
};

// Staging-write placement of the 16-byte piece loaded by lane l of a wave-wide
// load over a tile with PPR pieces per row: each group of 16 lanes writes 8 rows
// x 2 pieces when PPR <= 8 (with the stride above, distinct banks), else a
// contiguous part of one row.
template <int PPR>
__device__ __forceinline__ void piece_of(int l, int& row, int& piece) {
    if constexpr (PPR >= 16) {
        row = l / PPR;
        piece = l % PPR;
    } else {
        constexpr int LOG = PPR == 8 ? 3 : PPR == 4 ? 2 : PPR == 2 ? 1 : 0;
        piece = (l >> 3) & (PPR - 1);
        row = (l & 7) + 8 * (l >> (3 + LOG));
    }
}

template <int C, int NWK, int TV, int U, int GK>
struct StateLayout {
    static constexpr bool GLA = GK == kGateChannel, SCL = GK == kGateScalar;
    static constexpr int DKB = 16 * NWK, DVB = 16 * TV;
    static constexpr int KS = tile_stride(DKB);   // bf16 row stride of staged keys
    static constexpr int VS = tile_stride(DVB);   // bf16 row stride of staged values
    static constexpr int GS = DKB + 4;            // fp32 row stride of staged raw gates
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int KCH = al(C * KS * 2), VCH = al(C * VS * 2);
    static constexpr int GCH = GLA ? al(C * GS * 4) : SCL ? al(C * 4) : 0;   // raw gates (log2 units)
    static constexpr int CH = KCH + VCH + GCH;    // one staged chunk
    static constexpr int BUF = U * CH;            // one staged group
    static constexpr int bytes = 2 * BUF;
    static constexpr bool fits = bytes <= 160 * 1024;
};

template <int C, int DK, int NWK, int NWV, int TV, int U, int GK, bool REV = false>
__global__ __launch_bounds__(64 * NWK * NWV)
void state_kernel(StateParams p) {
    using Lay = StateLayout<C, NWK, TV, U, GK>;
    constexpr bool GLA = GK == kGateChannel, SCL = GK == kGateScalar;
    static_assert(Lay::fits, "LDS budget exceeded");
    static_assert(TV % NWV == 0, "value tiles split evenly over the wave groups");
    constexpr int NW = NWK * NWV, NT = 64 * NW, DKB = Lay::DKB, DVB = Lay::DVB;
    constexpr int TVW = TV / NWV;   // value tiles per wave
    constexpr int KS = Lay::KS, VS = Lay::VS, GS = Lay::GS;
    constexpr int CT = C / 16, JB = (CT + 1) / 2;
    constexpr int KP = C * DKB / 8, KP_PER = (KP + NT - 1) / NT;   // 16-byte key pieces per chunk
    constexpr int VP = C * DVB / 8, VP_PER = (VP + NT - 1) / NT;   // 16-byte value pieces
    constexpr int GP = GLA ? C * DKB / 4 : 0;                      // 16-byte gate pieces
    constexpr int GP_PER = GLA ? (GP + NT - 1) / NT : 0;

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    auto chunk_base = [&](int b, int u) { return smem + b * Lay::BUF + u * Lay::CH; };
    auto sK = [&](int b, int u) { return reinterpret_cast<u16*>(chunk_base(b, u)); };
    auto sV = [&](int b, int u) { return reinterpret_cast<u16*>(chunk_base(b, u) + Lay::KCH); };
    auto sG = [&](int b, int u) { return reinterpret_cast<float*>(chunk_base(b, u) + Lay::KCH + Lay::VCH); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = wave % NWK;      // key tile of this wave
    const int vgrp = wave / NWK;   // value tiles vgrp, vgrp + NWV, ...
    const int r16 = lane & 15, g = lane >> 4;

    const int L = logical_block_of(blockIdx.x, gridDim.x, p.remap);
    const int per_head = p.vblocks * p.kblocks;
    const int bh = L / per_head, rem = L % per_head;
    const int v0 = (rem / p.kblocks) * DVB, k0 = (rem % p.kblocks) * DKB;
    const int h = bh % p.H;
    const int T = p.T, dv = p.dv, NC = p.NC;
    const int NG = (NC + U - 1) / U;
    const int64_t tok0 = static_cast<int64_t>(bh) * T;
    const u16* kg = p.k + tok0 * DK + k0;
    const u16* vg = p.v + tok0 * dv + v0;
    const float* gg = GLA ? p.gate + tok0 * DK + k0 : nullptr;
    const float* gsc = SCL ? p.gate + tok0 : nullptr;
    const float lg2 = (GK == kGateFixed) ? p.gate[h] * kLog2e : 0.f;

    // sacc[t][r] = S[v0 + 16 tv(t) + r16][k0 + 16w + 4g + r], tv(t) = vgrp + NWV t
    f32x4 sacc[TVW];
    {
        const float* s0 = p.s0 ? p.s0 + (static_cast<int64_t>(bh) * dv + v0 + 16 * vgrp + r16) * DK + k0 + 16 * w + 4 * g
                               : nullptr;
#pragma unroll
        for (int t = 0; t < TVW; ++t) sacc[t] = s0 ? ldf4(s0 + 16 * NWV * t * DK) : zf4();
    }

    auto chunk_len = [&](int c) { return (T - c * C < C) ? (T - c * C) : C; };
    // chunk of the sequence at walk position c (the walk runs backwards with REV), and its
    // length (<= 0 past the end of the walk)
    auto phys = [&](int c) { return REV ? NC - 1 - c : c; };
    auto walk_len = [&](int c) { return c < NC ? chunk_len(phys(c)) : T - c * C; };

    // 16-byte pieces: wave `wave` covers a block of rows per load; piece_of places
    // them so that the staging writes are free of bank conflicts
    constexpr int KPPR = DKB / 8, VPPR = DVB / 8;
    constexpr int KRPW = 64 / KPPR, VRPW = 64 / VPPR;              // rows per wave-wide load
    auto key_piece = [&](int i, int& j, int& pc) {
        piece_of<KPPR>(lane, j, pc);
        j += KRPW * (wave + NW * i);
    };
    auto value_piece = [&](int i, int& j, int& pc) {
        piece_of<VPPR>(lane, j, pc);
        j += VRPW * (wave + NW * i);
    };
    auto key_ok = [&](int i) { return KP % NT == 0 || tid + i * NT < KP; };
    auto value_ok = [&](int i) { return VP % NT == 0 || tid + i * NT < VP; };

    // ---- two-slot register ring of raw 16-byte pieces, one group per slot
    u16x8 rk[2][U][KP_PER], rv[2][U][VP_PER];
    f32x4 rg[2][U][GLA ? GP_PER : 1];
    float rs[2][U];   // scalar gates: thread t < C holds token t's

    // Loads only: chunks past the last are clamped to it, rows past the end read
    // row 0; the zeroing happens where the data is consumed, so that no instruction
    // waits for a load before the data is needed.
    auto fetch = [&](int slot, int grp) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c_req = grp * U + u;
            const int c = phys(c_req < NC ? c_req : NC - 1);
            const int n = chunk_len(c);
            const u16* kc = kg + static_cast<int64_t>(c) * C * DK;
            const u16* vc = vg + static_cast<int64_t>(c) * C * dv;
#pragma unroll
            for (int i = 0; i < KP_PER; ++i) {
                int j, pc;
                key_piece(i, j, pc);
                const bool ok = key_ok(i) && j < n;
                rk[slot][u][i] = *reinterpret_cast<const u16x8*>(kc + (ok ? static_cast<unsigned>(j * DK + 8 * pc) : 0u));
            }
#pragma unroll
            for (int i = 0; i < VP_PER; ++i) {
                int j, pc;
                value_piece(i, j, pc);
                const bool ok = value_ok(i) && j < n;
                rv[slot][u][i] = *reinterpret_cast<const u16x8*>(vc + (ok ? static_cast<unsigned>(j * dv + 8 * pc) : 0u));
            }
            if constexpr (SCL) rs[slot][u] = gsc[static_cast<int64_t>(c) * C + (tid < n ? tid : 0)];
            if constexpr (GLA) {
                const float* gc = gg + static_cast<int64_t>(c) * C * DK;
#pragma unroll
                for (int i = 0; i < GP_PER; ++i) {
                    const int idx = tid + i * NT;
                    const int j = idx / (DKB / 4), col = (idx % (DKB / 4)) * 4;
                    const bool ok = idx < GP && j < n;
                    rg[slot][u][i] = ldf4(gc + (ok ? static_cast<unsigned>(j * DK + col) : 0u));
                }
            }
        }
    };

    // group grp (register slot) -> LDS buffer b, rows past the end zero
    auto stage = [&](int b, int slot, int grp) {
        const u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int n = walk_len(grp * U + u);   // <= 0 past the last chunk: all zero
            u16* ks = sK(b, u);
            u16* vs = sV(b, u);
#pragma unroll
            for (int i = 0; i < KP_PER; ++i) {
                if (key_ok(i)) {
                    int j, pc;
                    key_piece(i, j, pc);
                    *reinterpret_cast<u16x8*>(ks + j * KS + 8 * pc) = (j < n) ? rk[slot][u][i] : z;
                }
            }
#pragma unroll
            for (int i = 0; i < VP_PER; ++i) {
                if (value_ok(i)) {
                    int j, pc;
                    value_piece(i, j, pc);
                    *reinterpret_cast<u16x8*>(vs + j * VS + 8 * pc) = (j < n) ? rv[slot][u][i] : z;
                }
            }
            if constexpr (SCL) {
                if (tid < C) sG(b, u)[tid] = (tid < n) ? rs[slot][u] * kLog2e : 0.f;
            }
            if constexpr (GLA) {
                float* gs = sG(b, u);
#pragma unroll
                for (int i = 0; i < GP_PER; ++i) {
                    const int idx = tid + i * NT;
                    if (GP % NT == 0 || idx < GP) {
                        const int j = idx / (DKB / 4), col = (idx % (DKB / 4)) * 4;
                        stf4(gs + j * GS + col, (j < n) ? rg[slot][u][i] * kLog2e : zf4());
                    }
                }
            }
        }
    };

    // retention: carry weights g^(n-1-j) of this lane's tokens 16q + 4g + e, and g^n
    auto ret_weights = [&](int n, f32x4* wq, f32x4& dec) {
#pragma unroll
        for (int q = 0; q < CT; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * q + 4 * g + e;
                wq[q][e] = (j < n) ? ex2(static_cast<float>(REV ? j + 1 : n - 1 - j) * lg2) : 0.f;
            }
        const float d = ex2(static_cast<float>(n) * lg2);
        dec[0] = d; dec[1] = d; dec[2] = d; dec[3] = d;
    };
    f32x4 wfull[GK == kGateFixed ? CT : 1], dfull;   // full-chunk values (only the last chunk is shorter)
    if constexpr (GK == kGateFixed) ret_weights(C, wfull, dfull);

    // scalar gates: the chunk's inclusive cumulative log2-gates G by a wave prefix
    // scan (lane = token; padded tokens carry 0), carry weights e^(G_last - G_j) of
    // this lane's tokens 16q + 4g + e by shuffles, and the decay e^(G_last)
    auto scalar_weights = [&](const float* gs, f32x4* wq, f32x4& dec) {
        const float G = wave_inclusive_scan(lane < C ? gs[lane] : 0.f);
        const float last = __shfl(G, C - 1, 64);
#pragma unroll
        for (int q = 0; q < CT; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float gj = __shfl(G, 16 * q + 4 * g + e, 64);
                wq[q][e] = ex2(REV ? gj : last - gj);
            }
        const float d = ex2(last);
        dec[0] = d; dec[1] = d; dec[2] = d; dec[3] = d;
    };

    // GLA: carry weights e^(b_last - b_j) (REV: e^(b_j)) of this lane's tokens for key
    // channel k0 + 16w + r16, and the decays e^(b_last) of key channels 16w + 4g + r
    auto gla_weights = [&](const float* gs, f32x4* wq, f32x4& dec) {
        float tot[CT], exc[CT];
#pragma unroll
        for (int q = 0; q < CT; ++q) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = gs[(16 * q + 4 * g + e) * GS + 16 * w + r16];
            x[1] += x[0];
            x[2] += x[1];
            x[3] += x[2];
            wq[q] = x;
            float inc = x[3];
            float y = __shfl_up(inc, 16, 64);
            if (g >= 1) inc += y;
            y = __shfl_up(inc, 32, 64);
            if (g >= 2) inc += y;
            exc[q] = inc - x[3];
            tot[q] = __shfl(inc, 48 + r16, 64);
        }
        float run = 0.f;
#pragma unroll
        for (int q = 0; q < CT; ++q) {
            wq[q] = wq[q] + (run + exc[q]);   // b_j of token 16q + 4g + e
            run += tot[q];
        }
#pragma unroll
        for (int q = 0; q < CT; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) wq[q][e] = ex2(REV ? wq[q][e] : run - wq[q][e]);
#pragma unroll
        for (int r = 0; r < 4; ++r) dec[r] = ex2(__shfl(run, 4 * g + r, 64));
    };

    // snapshot values of the memory entering the latest valid chunk (bf16)
    bf16x4 snap[TVW];
#pragma unroll
    for (int t = 0; t < TVW; ++t) snap[t] = cvt4(sacc[t]);
    auto store_snap = [&](int c) {
        u16* st = p.states + ((static_cast<int64_t>(bh) * NC + c) * dv + v0 + 16 * vgrp + r16) * DK + k0 + 16 * w + 4 * g;
#pragma unroll
        for (int t = 0; t < TVW; ++t) st4(st + 16 * NWV * t * DK, snap[t]);
    };

    // the U chunks of group grp from LDS buffer b: contributions first (independent
    // MFMA chains), then in order: store the entering memory, S <- decay . S + dS.
    auto carry = [&](int b, int grp) {
        f32x4 ds[U][TVW];
        f32x4 dec[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = grp * U + u;
            if (c < NC) {
                const int n = walk_len(c);
                f32x4 wq[CT];
                if constexpr (GLA) {
                    gla_weights(sG(b, u), wq, dec[u]);
                } else if constexpr (SCL) {
                    scalar_weights(sG(b, u), wq, dec[u]);
                } else if (n == C) {
#pragma unroll
                    for (int q = 0; q < CT; ++q) wq[q] = wfull[q];
                    dec[u] = dfull;
                } else {
                    ret_weights(n, wq, dec[u]);
                }
                const u16* ks = sK(b, u);
                const u16* vs = sV(b, u);
                bf16x8 ka[JB];
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    const bool hi = 2 * jb + 1 < CT;
                    const bf16x4 lo4 = scale4(tr_op<KS>(ks, 32 * jb, 16 * w, r16, g), wq[2 * jb]);
                    const bf16x4 hi4 = hi ? scale4(tr_op<KS>(ks, 32 * jb + 16, 16 * w, r16, g), wq[(2 * jb + 1) % CT])
                                          : zero4();
                    ka[jb] = join8(lo4, hi4);
                }
#pragma unroll
                for (int t = 0; t < TVW; ++t) {
                    f32x4 acc = zf4();
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb)
                        acc = mfma_16x16x32(ka[jb], tr_split<VS>(vs, jb, 16 * (vgrp + NWV * t), 2 * jb + 1 < CT, r16, g),
                                            acc);
                    ds[u][t] = acc;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = grp * U + u;
            if (c < NC) {
#pragma unroll
                for (int t = 0; t < TVW; ++t) snap[t] = cvt4(sacc[t]);
#pragma unroll
                for (int t = 0; t < TVW; ++t) sacc[t] = sacc[t] * dec[u] + ds[u][t];
            }
            if (c < NC) store_snap(phys(c));
        }
    };

    if (NC > 0) {
        // prologue: groups 0 and 1 in the ring, group 0 staged, group 2 requested
        fetch(0, 0);
        fetch(1, 1);
        stage(0, 0, 0);
        fetch(0, 2);
        lds_barrier();
        for (int g0 = 0; g0 < NG; g0 += 2) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int grp = g0 + s;
                if (grp < NG) {
                    carry(s, grp);
                    if (grp + 1 < NG) stage(s ^ 1, s ^ 1, grp + 1);
                    fetch(s ^ 1, grp + 3);   // slot of group grp+1 is free again (clamped past the end)
                    lds_barrier();
                }
            }
        }
    }

    if (p.s_out) {
        float* so = p.s_out + (static_cast<int64_t>(bh) * dv + v0 + 16 * vgrp + r16) * DK + k0 + 16 * w + 4 * g;
#pragma unroll
        for (int t = 0; t < TVW; ++t) stf4(so + 16 * NWV * t * DK, sacc[t]);
    }
}

}  // namespace ck
}  // namespace glr
