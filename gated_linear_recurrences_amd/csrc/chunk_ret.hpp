// Retention (fixed decay per head), chunked forward, bf16 storage - software-pipelined.
//
// Method: the chunkwise form of retention ("Le architetture lineari: RetNet,
// RWKV, xLSTM", section "RetNet: la retention e le sue tre forme", Fig. 16.5)
// with S_t = g S_{t-1} + v_t k_t^T, o_t = S_t q_t. Per chunk of n tokens, with
// local index i, j and incoming memory S_in:
//   P_ij  = g^(i-j) (q_i.k_j)  (j <= i)
//   o_i   = sum_j P_ij v_j + g^(i+1) S_in q_i
//   S_out = g^n S_in + sum_j k_j (g^(n-1-j) v_j)^T      (as S^T)
//
// Decomposition (gfx950): a workgroup owns one (batch, head) and DVT = 16 MT value
// channels (rows of S evolve independently); MT * KS waves split its slice of
// S^T by value tile (mt) and key range (ks), each keeping a d_k/KS x 16 block in
// MFMA accumulators. Waves own output row tiles it with it % KS == ks.
//
// Pipeline: two LDS buffers of staged tokens and of P. Iteration c has two
// intervals separated by workgroup barriers:
//   I   outputs of chunk c (P V + readout), the carry of chunk c (each wave its
//       own key tiles), publication of the new memory in bf16, staging of chunk
//       c+1 from registers into the other buffer, and the HBM prefetch of chunk
//       c+2 into registers;
//   II  the triangle P of chunk c+1 (tiles go first to waves that own no output
//       tile) and the readout of the memory for chunk c+1.
// Only two barriers per chunk; staging, HBM traffic and the triangle of the next
// chunk overlap the outputs and carry of the current one. Operands that reduce
// over tokens are read from token-major LDS with ds_read_b64_tr_b16; the carry
// weights g^(n-1-j) are folded into a copy of the (small) v tile.
#pragma once

#include "chunk_common.hpp"

namespace glr {
namespace ck {

template <int C, int DK, int MT, int KS>
struct RetLayout {
    static constexpr int NW = MT * KS;
    static constexpr int DVT = 16 * MT;
    static constexpr int QS = DK + 8;   // token-major q, k row stride
    static constexpr int VS = DVT + 8;  // token-major v row stride
    static constexpr int TS = C + 8;    // P row stride
    static constexpr int SS = DK + 8;   // published S^T: one row per value channel
    static constexpr int OS = 24;       // output staging row stride
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int oQ = 0;
    static constexpr int oK = al(oQ + C * QS * 2);
    static constexpr int oV = al(oK + C * QS * 2);
    static constexpr int oVw = al(oV + C * VS * 2);
    static constexpr int SET = al(oVw + C * VS * 2);        // one staged buffer
    static constexpr int oP = 2 * SET;
    static constexpr int PSZ = al(C * TS * 2);
    static constexpr int oS = oP + 2 * PSZ;
    static constexpr int oO = al(oS + DVT * SS * 2);
    static constexpr int bytes = al(oO + NW * 16 * OS * 2);
    static_assert(bytes <= 160 * 1024, "LDS budget exceeded");
};

template <int C, int DK, int MT, int KS>
__global__ __launch_bounds__(64 * MT * KS)
void retention_kernel(Params p) {
    using Lay = RetLayout<C, DK, MT, KS>;
    constexpr int NW = Lay::NW, NT = 64 * NW, DVT = Lay::DVT;
    constexpr int CT = C / 16, KT = DK / 16;
    static_assert(KT % KS == 0, "key split must divide the key tiles");
    constexpr int KTW = KT / KS, KB = (KT + 1) / 2, JB = (CT + 1) / 2;
    constexpr int QS = Lay::QS, VS = Lay::VS, TS = Lay::TS, SS = Lay::SS, OS = Lay::OS;

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    auto sQ = [&](int b) { return reinterpret_cast<u16*>(smem + b * Lay::SET + Lay::oQ); };
    auto sK = [&](int b) { return reinterpret_cast<u16*>(smem + b * Lay::SET + Lay::oK); };
    auto sV = [&](int b) { return reinterpret_cast<u16*>(smem + b * Lay::SET + Lay::oV); };
    auto sVw = [&](int b) { return reinterpret_cast<u16*>(smem + b * Lay::SET + Lay::oVw); };
    auto sP = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oP + b * Lay::PSZ); };
    u16* const sS = reinterpret_cast<u16*>(smem + Lay::oS);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mt = w % MT, ks = w / MT, ct0 = ks * KTW;
    const int r16 = lane & 15, g = lane >> 4;
    u16* const so = reinterpret_cast<u16*>(smem + Lay::oO) + w * 16 * OS;

    const int L = logical_block(p);
    const int bh = L / p.tiles, v0 = (L % p.tiles) * DVT, h = bh % p.H;
    const int T = p.T, dv = p.dv;
    const int64_t tok0 = static_cast<int64_t>(bh) * T;
    const u16* qg = p.q + tok0 * DK;
    const u16* kg = p.k + tok0 * DK;
    const u16* vg = p.v + tok0 * dv + v0;
    u16* og = p.o + tok0 * dv + v0;
    const float lg2 = p.gate[h] * kLog2e;

    // this lane's output scales g^(i+1), rows i = 16it + 4g + r
    f32x4 oscale[CT];
#pragma unroll
    for (int it = 0; it < CT; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) oscale[it][r] = ex2(static_cast<float>(16 * it + 4 * g + r + 1) * lg2);

    // the wave's block of the memory: sacc[t][r] = S[v0 + 16mt + r16][16(ct0+t) + 4g + r]
    f32x4 sacc[KTW];
    {
        const float* srow = p.s0 ? p.s0 + (static_cast<int64_t>(bh) * dv + v0 + 16 * mt + r16) * DK : nullptr;
#pragma unroll
        for (int t = 0; t < KTW; ++t) sacc[t] = srow ? ldf4(srow + 16 * (ct0 + t) + 4 * g) : zf4();
    }

    // ---- register staging: 4-row micro-tiles of QV columns
    constexpr int QV = ((C / 4) * (DK / 8) >= NT) ? 8 : 4;
    typedef typename Vec<QV>::type qv_t;
    constexpr int QK_ITEMS = (C / 4) * (DK / QV), QK_PER = (QK_ITEMS + NT - 1) / NT;
    constexpr int V_ITEMS = (C / 4) * (DVT / 8), V_PER = (V_ITEMS + NT - 1) / NT;
    qv_t rq[QK_PER][4], rk[QK_PER][4];
    u16x8 rv[V_PER][4];

    auto chunk_len = [&](int c) { return (T - c * C < C) ? (T - c * C) : C; };

    auto fetch = [&](int c) {
        const int n = chunk_len(c);
        const u16* qc = qg + static_cast<int64_t>(c) * C * DK;
        const u16* kc = kg + static_cast<int64_t>(c) * C * DK;
        const u16* vc = vg + static_cast<int64_t>(c) * C * dv;
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
    };

    auto stage = [&](int b, int c) {
        const int n = chunk_len(c);
        u16* q_ = sQ(b);
        u16* k_ = sK(b);
        u16* v_ = sV(b);
        u16* vw_ = sVw(b);
#pragma unroll
        for (int pi = 0; pi < QK_PER; ++pi) {
            const int item = tid + pi * NT;
            if (item < QK_ITEMS) {
                const int row0 = (item / (DK / QV)) * 4, col0 = (item % (DK / QV)) * QV;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    *reinterpret_cast<qv_t*>(q_ + (row0 + rr) * QS + col0) = rq[pi][rr];
                    *reinterpret_cast<qv_t*>(k_ + (row0 + rr) * QS + col0) = rk[pi][rr];
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
                    const int j = row0 + rr;
                    *reinterpret_cast<u16x8*>(v_ + j * VS + col0) = rv[pi][rr];
                    // the carry weight g^(n-1-j) of token j, folded into the v tile
                    const float wgt = (j < n) ? ex2(static_cast<float>(n - 1 - j) * lg2) : 0.f;
                    u16x8 t;
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = bits(static_cast<__bf16>(bf16_bits_to_f32(rv[pi][rr][e]) * wgt));
                    *reinterpret_cast<u16x8*>(vw_ + j * VS + col0) = t;
                }
            }
        }
    };

    // the wave's block of S^T in bf16, one row per value channel
    auto publish = [&]() {
#pragma unroll
        for (int t = 0; t < KTW; ++t) st4(sS + (16 * mt + r16) * SS + 16 * (ct0 + t) + 4 * g, cvt4(sacc[t]));
    };

    // the decayed triangle of buffer b; pair tiles go first to the waves that own no
    // output tile (the highest wave ids)
    auto phase1 = [&](int b) {
        constexpr int NPAIR = CT * (CT + 1) / 2;
        constexpr int NQ = (NPAIR + NW - 1) / NW;
        const u16* q_ = sQ(b);
        const u16* k_ = sK(b);
        u16* p_ = sP(b);
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
            const int pr = (NW - 1 - w) + NW * qq;
            if (pr < NPAIR) {
                int it, jt;
                pair_of(pr, it, jt);
                const int i = 16 * it + r16;
                f32x4 acc = zf4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    acc = mfma_16x16x32(split_op<KT, QS>(k_, 16 * jt + r16, kb, g), split_op<KT, QS>(q_, i, kb, g), acc);
                // acc[r] = q_i . k_j with j = 16jt + 4g + r
                bf16x4 pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jt + 4 * g + r;
                    const float val = acc[r] * ex2(static_cast<float>(i - j) * lg2);
                    pv[r] = static_cast<__bf16>((j <= i) ? val : 0.f);
                }
                st4(p_ + i * TS + 16 * jt + 4 * g, pv);
            }
        }
    };

    // readout of the published memory for the owned row tiles of buffer b
    f32x4 oe[CT];
    auto readout = [&](int b) {
        const u16* q_ = sQ(b);
        const u16* srow = sS + (16 * mt + r16) * SS;
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            if (it % KS != ks) continue;
            f32x4 acc = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 sb = join8(ld4(srow + 32 * kb + 4 * g),
                                        (2 * kb + 1 < KT) ? ld4(srow + 32 * kb + 16 + 4 * g) : zero4());
                acc = mfma_16x16x32(split_op<KT, QS>(q_, 16 * it + r16, kb, g), sb, acc);
            }
            oe[it] = acc;
        }
    };

    // outputs of the owned row tiles of chunk c (buffer b): P V + g^(i+1) S_in q_i
    auto outputs = [&](int b, int c) {
        const int n = chunk_len(c);
        const u16* p_ = sP(b);
        const u16* v_ = sV(b);
        u16* oc = og + static_cast<int64_t>(c) * C * dv;
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            if (it % KS != ks) continue;
            f32x4 oi = zf4();
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                if (2 * jb <= it) {
                    const bool hi = 2 * jb + 1 <= it;
                    const u16* prow = p_ + (16 * it + r16) * TS + 32 * jb + 4 * g;
                    oi = mfma_16x16x32(join8(ld4(prow), hi ? ld4(prow + 16) : zero4()),
                                       tr_split<VS>(v_, jb, 16 * mt, hi, r16, g), oi);
                }
            }
            bf16x4 res = cvt4(oi + oscale[it] * oe[it]);
#pragma unroll
            for (int r = 0; r < 4; ++r) so[(4 * g + r) * OS + r16] = bits(res[r]);
            if (lane < 32) {
                const int row = lane >> 1, half = lane & 1;
                const u16x8 val = *reinterpret_cast<const u16x8*>(so + row * OS + 8 * half);
                if (16 * it + row < n)
                    *reinterpret_cast<u16x8*>(oc + static_cast<unsigned>((16 * it + row) * dv + 16 * mt + 8 * half)) = val;
            }
        }
    };

    // the carry of chunk c: S^T <- g^n S^T + K^T (w v) on the wave's key tiles
    auto carry = [&](int b, int c) {
        const int n = chunk_len(c);
        const float dec = ex2(static_cast<float>(n) * lg2);
        const u16* k_ = sK(b);
        const u16* vw_ = sVw(b);
#pragma unroll
        for (int t = 0; t < KTW; ++t) {
            f32x4 acc = sacc[t] * dec;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                const bool hi = 2 * jb + 1 < CT;
                acc = mfma_16x16x32(tr_split<QS>(k_, jb, 16 * (ct0 + t), hi, r16, g),
                                    tr_split<VS>(vw_, jb, 16 * mt, hi, r16, g), acc);
            }
            sacc[t] = acc;
        }
    };

    const int NC = (T + C - 1) / C;
    if (NC > 0) {
        fetch(0);
        stage(0, 0);
        publish();
        if (NC > 1) fetch(1);
        lds_barrier();
        phase1(0);
        readout(0);
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            const int b = c & 1;
            // interval I
            outputs(b, c);
            carry(b, c);
            publish();
            if (c + 1 < NC) stage(b ^ 1, c + 1);
            if (c + 2 < NC) fetch(c + 2);
            lds_barrier();
            // interval II
            if (c + 1 < NC) {
                phase1(b ^ 1);
                readout(b ^ 1);
            }
            lds_barrier();
        }
    }

    if (p.s_out) {
        float* srow = p.s_out + (static_cast<int64_t>(bh) * dv + v0 + 16 * mt + r16) * DK;
#pragma unroll
        for (int t = 0; t < KTW; ++t) stf4(srow + 16 * (ct0 + t) + 4 * g, sacc[t]);
    }
}

template <int C, int DK, int MT, int KS>
hipError_t launch_retention_cfg(const ChunkArgs& a, hipStream_t stream) {
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
    p.tiles = a.dv / (16 * MT);
    const int64_t G = static_cast<int64_t>(a.B) * a.H * p.tiles;
    p.remap = (G % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((retention_kernel<C, DK, MT, KS>), dim3(static_cast<unsigned>(G)), dim3(64 * MT * KS), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace ck
}  // namespace glr
