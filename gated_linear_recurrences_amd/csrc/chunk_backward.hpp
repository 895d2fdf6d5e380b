// Backward of the chunked forward for the fixed (retention) and scalar data-dependent
// decays, bf16 storage.
//
// Method: reverse-mode differentiation of the recurrence S_t = a_t S_{t-1} + v_t k_t^T,
// o_t = S_t q_t ("Scrivere meglio nella memoria", section "Dimenticare: i gate", scalar
// decay), organised like the chunkwise forward of the RetNet page (section "RetNet: la
// retention e le sue tre forme"): per chunk a decayed triangle, between chunks a carried
// d_v x d_k matrix. With chunk-local inclusive cumulative log-gates G, M_ij = e^(G_i - G_j)
// for j <= i (else 0), S_in the memory entering the chunk and R the gradient of the loss
// with respect to the memory at the chunk's last token:
//   dq_i = sum_{j<=i} M_ij (do_i . v_j) k_j + e^(G_i) S_in^T do_i
//   dk_j = sum_{i>=j} M_ij (do_i . v_j) q_i + e^(G_last - G_j) R^T v_j
//   dv_j = sum_{i>=j} M_ij (q_i . k_j) do_i + e^(G_last - G_j) R k_j
// and, since every term of o_t carries e^(B_t) and every write of token j carries
// e^(-B_j) (B the cumulative log-gate over the sequence), the gate's gradient is
//   d log a_t = sum_{s >= t} (q_s . dq_s - k_s . dk_s) + <dS_T, S_T>.
// The call runs four passes: the forward state pass (snapshots S_in, final memory),
// the same pass walked backwards on (q, dO) (snapshots R, gradient of S_0), the
// gradient pass below (chunk-parallel), and the gate pass (one kernel per sequence,
// plus a sum over the batch for a fixed gate).
//
// Gradient pass (gfx950): persistent workgroups of eight waves, one per CU, each taking
// (sequence, chunk) items in turn and loading the next item's operands into registers
// while the current one computes. q, k, v,
// dO are staged token-major; A1 = (Q K^T) . M and A2 = (dO V^T) . M are formed on MFMA
// into LDS (bf16, all C/16 x C/16 tiles, the upper ones zero). Every product is computed
// transposed - feature rows, token columns - so that a lane ends with four consecutive
// features of one token (one 8-byte store):
//   dV^T = dO^T A1 + R K^T diag(w)      dK^T = Q^T A2 + R^T V^T diag(w)
//   dQ^T = K^T A2^T + S_in^T dO^T diag(e^G),     w_j = e^(G_last - G_j),
// with the operands read transposed (ds_read_b64_tr_b16) or by rows as each needs; the
// staged tiles use the chunk-swizzled layout (SwzTile) so that both kinds of read are
// free of bank conflicts.
// R and then S_in take turns in one LDS region. The per-token sums q.dq and k.dk meet
// in LDS: per feature tile a partial (reduced over the lane group), added in tile order
// (no atomics: the gradients are bit-for-bit repeatable).
#pragma once

#include "chunk_common.hpp"
#include "chunk_two_pass.hpp"

namespace glr {
namespace ck {

struct GradParams {
    const u16* q;          // [BH][T][DK]
    const u16* k;          // [BH][T][DK]
    const u16* v;          // [BH][T][DV]
    const u16* dout;       // [BH][T][DV]
    const float* gate;     // fixed: log gamma [H]; scalar: log alpha [BH][T]
    const u16* s_in;       // [BH][NC][DV][DK] forward snapshots
    const u16* r;          // [BH][NC][DV][DK] backward snapshots
    u16* dq;               // [BH][T][DK]
    u16* dk;               // [BH][T][DK]
    u16* dv;               // [BH][T][DV]
    float* gq;             // [BH][T]: q.dq - k.dk per token
    int H, T, NC;
    int items;             // BH * NC (sequence, chunk) pairs
};

template <int C, int DK, int DV>
struct GradLayout {
    using TQ = SwzTile<DK>;   // q, k and the memories (rows of d_k)
    using TV = SwzTile<DV>;   // v and dO
    using TA = SwzTile<C>;    // A1, A2
    static constexpr int QS = TQ::STRIDE, VS = TV::STRIDE, AS = TA::STRIDE, XS = TQ::STRIDE;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + al(C * QS * 2);
    static constexpr int oV = oK + al(C * QS * 2);
    static constexpr int oO = oV + al(C * VS * 2);
    static constexpr int oA1 = oO + al(C * VS * 2);
    static constexpr int oA2 = oA1 + al(C * AS * 2);
    static constexpr int oX = oA2 + al(C * AS * 2);     // R, then S_in ([DV][DK])
    static constexpr int oG = oX + al(DV * XS * 2);
    static constexpr int oQD = oG + al(C * 4);              // [DK / 16][C] partial q . dq
    static constexpr int oKD = oQD + al(DK / 16 * C * 4);   // [DK / 16][C] partial k . dk
    static constexpr int bytes = oKD + al(DK / 16 * C * 4);
    static_assert(bytes <= 160 * 1024, "LDS budget of the gradient pass exceeded");
};

template <int C, int DK, int DV, int GK>
__global__ __launch_bounds__(512)
void grad_kernel(GradParams p) {
    using Lay = GradLayout<C, DK, DV>;
    constexpr int NT = 512, NW = 8;
    constexpr int CT = C / 16, JB = (CT + 1) / 2;
    using TQ = typename Lay::TQ;
    using TV = typename Lay::TV;
    using TA = typename Lay::TA;
    constexpr int KB = (DK + 31) / 32, VB = (DV + 31) / 32;
    constexpr int QP = C * DK / 8, QP_PER = (QP + NT - 1) / NT;
    constexpr int VP = C * DV / 8, VP_PER = (VP + NT - 1) / NT;
    constexpr int XP = DV * DK / 8, XP_PER = (XP + NT - 1) / NT;
    constexpr int FK = DK / 16, FV = DV / 16;
    static_assert(GK == kGateFixed || GK == kGateScalar, "fixed or scalar gates");

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sQ = reinterpret_cast<u16*>(smem + Lay::oQ);
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    u16* const sV = reinterpret_cast<u16*>(smem + Lay::oV);
    u16* const sO = reinterpret_cast<u16*>(smem + Lay::oO);
    u16* const sA1 = reinterpret_cast<u16*>(smem + Lay::oA1);
    u16* const sA2 = reinterpret_cast<u16*>(smem + Lay::oA2);
    u16* const sX = reinterpret_cast<u16*>(smem + Lay::oX);
    float* const sG = reinterpret_cast<float*>(smem + Lay::oG);
    float* const sQD = reinterpret_cast<float*>(smem + Lay::oQD);
    float* const sKD = reinterpret_cast<float*>(smem + Lay::oKD);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int T = p.T;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};

    // Persistent: this workgroup takes items (sequence, chunk) blockIdx.x, + gridDim.x, ...;
    // the next item's operands are loaded into registers while the current one computes.
    // Rows past the end of a sequence read row 0 and are zeroed on staging.
    u16x8 rq[QP_PER], rk[QP_PER], rv[VP_PER], ro[VP_PER], rx[XP_PER], rs[XP_PER];
    float rgate = 0.f;
    auto load_item = [&](int item) {
        const int lbh = item / p.NC, lc = item % p.NC;
        const int lt0 = lc * C, ln = (T - lt0 < C) ? (T - lt0) : C;
        const int64_t ltok0 = static_cast<int64_t>(lbh) * T + lt0;
        const int64_t lchunk = static_cast<int64_t>(lbh) * p.NC + lc;
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
#pragma unroll
        for (int i = 0; i < XP_PER; ++i) {
            const int idx = tid + i * NT;
            const unsigned off = (idx < XP) ? static_cast<unsigned>(idx * 8) : 0u;
            rx[i] = *reinterpret_cast<const u16x8*>(p.r + lchunk * DV * DK + off);
            rs[i] = *reinterpret_cast<const u16x8*>(p.s_in + lchunk * DV * DK + off);
        }
        if constexpr (GK == kGateScalar) rgate = (tid < ln) ? p.gate[ltok0 + tid] : 0.f;
    };

    int item = blockIdx.x;
    if (item >= p.items) return;
    load_item(item);
    for (;;) {
        const int bh = item / p.NC, c = item % p.NC;
        const int t0 = c * C, n = (T - t0 < C) ? (T - t0) : C;
        const int64_t tok0 = static_cast<int64_t>(bh) * T + t0;

        // ---- stage q, k, v, dO, R; cumulative gates (log2 units); zero the per-token sums
#pragma unroll
        for (int i = 0; i < QP_PER; ++i) {
            const int idx = tid + i * NT;
            if (idx < QP) {
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                *reinterpret_cast<u16x8*>(sQ + TQ::off(j, col)) = (j < n) ? rq[i] : z8;
                *reinterpret_cast<u16x8*>(sK + TQ::off(j, col)) = (j < n) ? rk[i] : z8;
            }
        }
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
        u16x8 rs_cur[XP_PER];
#pragma unroll
        for (int i = 0; i < XP_PER; ++i) rs_cur[i] = rs[i];
        const float gate_cur = rgate;
        const int step = static_cast<int>(gridDim.x);
        const int next = (item < p.items - step) ? item + step : p.items;
        if (next < p.items) load_item(next);   // in flight during this item's products
        if (w == 0) {
            float x;
            if constexpr (GK == kGateScalar) {
                x = wave_inclusive_scan(gate_cur * kLog2e);   // padded tokens add 0
            } else {
                const float lg2 = p.gate[bh % p.H] * kLog2e;
                x = static_cast<float>((lane < n ? lane : n - 1) + 1) * lg2;   // flat past the end
            }
            if (lane < C) sG[lane] = x;
        }
        lds_barrier();
        const float glast = sG[C - 1];

        // ---- A1 = (Q K^T) . M and A2 = (dO V^T) . M, every tile (upper ones zero):
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
                    }
                    acc = mfma_16x16x32(a8, b8, acc);
                }
                const float gi = sG[i];
                const f32x4 gj = ldf4(sG + 16 * jt + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int j = 16 * jt + 4 * g + r;
                    pv[r] = static_cast<__bf16>((j <= i) ? acc[r] * ex2(gi - gj[r]) : 0.f);
                }
            }
            st4(dst + TA::off(i, 16 * jt + 4 * g), pv);
        }
        lds_barrier();

        // transposed operand over 32 tokens (rows 32b .. 32b + 31) of a token-major array
        // X with row stride RS, column tile n0; the second half zero unless `hi`
        auto wq_of = [&](int j) { return ex2(glast - sG[j]); };

        // ---- dV^T and dK^T tiles: (feature tile, token tile jt); lane holds
        // D[f = 16 ft + 4g + r][j = 16 jt + r16]
        for (int t = w; t < (FV + FK) * CT; t += NW) {
            const bool isv = t < FV * CT;
            const int ft = (isv ? t : t - FV * CT) / CT, jt = (isv ? t : t - FV * CT) % CT;
            const int j = 16 * jt + r16;
            f32x4 acc = zf4(), acc2 = zf4();
            // term 1: sum over i >= j of X^T[f][i] A[i][j] (A1 with dO for dV, A2 with Q for dK)
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                if (32 * b + 31 < 16 * jt) continue;                 // rows i all above j
                const bool hi = 2 * b + 1 < CT;
                const bf16x8 xa = isv ? tr_split_s<DV>(sO, b, 16 * ft, hi, r16, g) : tr_split_s<DK>(sQ, b, 16 * ft, hi, r16, g);
                const bf16x8 ab = isv ? tr_split_s<C>(sA1, b, 16 * jt, hi, r16, g) : tr_split_s<C>(sA2, b, 16 * jt, hi, r16, g);
                acc = mfma_16x16x32(xa, ab, acc);
            }
            if (isv) {
                // term 2: sum over keys m of R[f][m] K[j][m] (rows of R and of K, natural order)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int col = rr_col(kb, g, KB);
                    bf16x8 xa = as_bf16x8(z8), kb8 = as_bf16x8(z8);
                    if (col < DK) {
                        xa = *reinterpret_cast<const bf16x8*>(sX + TQ::off(16 * ft + r16, col));
                        kb8 = *reinterpret_cast<const bf16x8*>(sK + TQ::off(j, col));
                    }
                    acc2 = mfma_16x16x32(xa, kb8, acc2);
                }
            } else {
                // term 2: sum over values m of R[m][f] V[j][m] (R read transposed, rows of V split
                // like the transposed operand)
#pragma unroll
                for (int b = 0; b < VB; ++b) {
                    const bool hi = 32 * b + 16 < DV;
                    const bf16x8 xa = tr_split_s<DK>(sX, b, 16 * ft, hi, r16, g);
                    const int vc = 32 * b + 4 * g;
                    const bf16x8 vb = join8(ld4(sV + TV::off(j, vc)), hi ? ld4(sV + TV::off(j, vc + 16)) : zero4());
                    acc2 = mfma_16x16x32(xa, vb, acc2);
                }
            }
            const float wj = wq_of(j);
            acc = acc + acc2 * wj;
            if (!isv) {
                // k_j . dk_j over this tile's features: the lane's four, then the lane group
                const f32x4 kj = up4(ld4(sK + TQ::off(j, 16 * ft + 4 * g)));
                float part = kj[0] * acc[0] + kj[1] * acc[1] + kj[2] * acc[2] + kj[3] * acc[3];
                part += __shfl_xor(part, 16, 64);
                part += __shfl_xor(part, 32, 64);
                if (g == 0) sKD[ft * C + j] = part;
            }
            if (j < n) {
                if (isv) st4(p.dv + (tok0 + j) * DV + 16 * ft + 4 * g, cvt4(acc));
                else st4(p.dk + (tok0 + j) * DK + 16 * ft + 4 * g, cvt4(acc));
            }
        }
        lds_barrier();   // R is dead: the region takes S_in
        stage_x(rs_cur);
        lds_barrier();

        // ---- dQ^T tiles: (key tile ft, token tile it); lane holds dQ[i = 16it + r16][f = 16ft + 4g + r]
        for (int t = w; t < FK * CT; t += NW) {
            const int ft = t / CT, it = t % CT;
            const int i = 16 * it + r16;
            f32x4 acc = zf4(), acc2 = zf4();
            // term 1: sum over j <= i of K[j][f] A2[i][j] (K transposed, rows of A2 split)
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                if (32 * b > 16 * it + 15) continue;                 // columns j all past i
                const bool hi = 2 * b + 1 < CT;
                const bf16x8 ka = tr_split_s<DK>(sK, b, 16 * ft, hi, r16, g);
                const int ac = 32 * b + 4 * g;
                acc = mfma_16x16x32(ka, join8(ld4(sA2 + TA::off(i, ac)), hi ? ld4(sA2 + TA::off(i, ac + 16)) : zero4()), acc);
            }
            // term 2: sum over values m of S_in[m][f] dO[i][m], scaled by e^(G_i)
#pragma unroll
            for (int b = 0; b < VB; ++b) {
                const bool hi = 32 * b + 16 < DV;
                const bf16x8 xa = tr_split_s<DK>(sX, b, 16 * ft, hi, r16, g);
                const int oc = 32 * b + 4 * g;
                acc2 = mfma_16x16x32(xa, join8(ld4(sO + TV::off(i, oc)), hi ? ld4(sO + TV::off(i, oc + 16)) : zero4()), acc2);
            }
            acc = acc + acc2 * ex2(sG[i]);
            const f32x4 qi = up4(ld4(sQ + TQ::off(i, 16 * ft + 4 * g)));
            float part = qi[0] * acc[0] + qi[1] * acc[1] + qi[2] * acc[2] + qi[3] * acc[3];
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            if (g == 0) sQD[ft * C + i] = part;
            if (i < n) st4(p.dq + (tok0 + i) * DK + 16 * ft + 4 * g, cvt4(acc));
        }
        lds_barrier();
        if (tid < n) {
            float qd = 0.f, kd = 0.f;
#pragma unroll
            for (int f = 0; f < FK; ++f) {
                qd += sQD[f * C + tid];
                kd += sKD[f * C + tid];
            }
            p.gq[tok0 + tid] = qd - kd;
        }
        // the next item's staging overwrites only regions every wave has finished reading
        // (the barrier above); the per-token sums it rewrites wait behind its own barriers
        if (next >= p.items) break;
        item = next;
    }
}

// Gate gradients from the per-token sums g_s = q_s.dq_s - k_s.dk_s, one workgroup of 256
// threads per sequence: scalar gates d log a_t = sum_{s>=t} g_s + <dS_T, S_T> (a reverse
// scan: each thread a contiguous run of tokens, run totals joined by wave scans and the
// four wave totals); a fixed gate the sequence's share sum_s (s + 1) g_s + T <dS_T, S_T>,
// left in g_0 of the sequence for gate_head_sum_kernel, which adds the batch up per head
// (in batch order: no atomics).
template <bool SCALAR>
__global__ __launch_bounds__(256)
void gate_grad_kernel(float* __restrict__ gq, const float* __restrict__ ds_out, const float* __restrict__ s_fin,
                      float* __restrict__ dgate, int T, int dsz) {
    __shared__ float wred[4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t bh = blockIdx.x;
    auto block_sum = [&](float x) {
        x = wave_sum(x);
        if (lane == 0) wred[w] = x;
        __syncthreads();
        const float r = wred[0] + wred[1] + wred[2] + wred[3];
        __syncthreads();
        return r;
    };
    float fin = 0.f;
    if (ds_out != nullptr) {
        const f32x4* a = reinterpret_cast<const f32x4*>(ds_out + bh * dsz);
        const f32x4* b = reinterpret_cast<const f32x4*>(s_fin + bh * dsz);
        float x = 0.f;
#pragma unroll 4
        for (int e = tid; e < dsz / 4; e += 256) {
            const f32x4 p = a[e], r = b[e];
            x += p[0] * r[0] + p[1] * r[1] + p[2] * r[2] + p[3] * r[3];
        }
        fin = block_sum(x);
    }
    float* g = gq + bh * T;
    const int per = (T + 255) / 256;
    const int lo = (tid * per < T) ? tid * per : T, hi = (lo + per < T) ? lo + per : T;
    if constexpr (SCALAR) {
        float run = 0.f;
        for (int t = lo; t < hi; ++t) run += g[t];
        // sum of the runs after this thread's: the rest of its wave, then the later waves
        const float incl = wave_inclusive_scan(run);
        const float wtot = __shfl(incl, 63, 64);
        if (lane == 0) wred[w] = wtot;
        __syncthreads();
        float after = wtot - incl;
        for (int u = w + 1; u < 4; ++u) after += wred[u];
        float acc = after + fin;
        for (int t = hi - 1; t >= lo; --t) {
            acc += g[t];
            dgate[bh * T + t] = acc;
        }
    } else {
        float x = 0.f;
        for (int t = lo; t < hi; ++t) x += static_cast<float>(t + 1) * g[t];
        const float part = block_sum(x) + static_cast<float>(T) * fin;
        if (tid == 0 && T > 0) g[0] = part;   // every read of g in this workgroup is done
    }
}

static __global__ __launch_bounds__(256)
void gate_head_sum_kernel(const float* __restrict__ gq, float* __restrict__ dgate, int B, int H, int T) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    float tot = 0.f;
    if (T > 0)
        for (int b = 0; b < B; ++b) tot += gq[(static_cast<int64_t>(b) * H + h) * T];
    dgate[h] = tot;
}

// ====================================================================== launch
// Workspace of a backward call: the forward and the backward snapshots
// ([BH][NC][DV][DK] bf16 each), the final memory [BH][DV][DK] fp32 and the per-token
// sums [BH][T] fp32, each from a 256-byte boundary.
inline size_t bwd_align(size_t x) { return (x + 255) / 256 * 256; }
inline size_t bwd_workspace_bytes(int64_t heads, int T, int chunk, int dk, int dv) {
    const int64_t nc = (T + chunk - 1) / chunk;
    return 2 * bwd_align(heads * nc * dv * dk * 2) + bwd_align(heads * dv * dk * 4) + bwd_align(heads * T * 4);
}

template <int C, int DK, int DV, int GK>
hipError_t launch_backward_dv(const BwdArgs& a, hipStream_t stream) {
    const int NC = (a.T + C - 1) / C;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    unsigned char* base = static_cast<unsigned char*>(a.ws);
    u16* fwd = reinterpret_cast<u16*>(base);
    u16* rev = reinterpret_cast<u16*>(base + bwd_align(heads * NC * DV * DK * 2));
    float* sfin = reinterpret_cast<float*>(base + 2 * bwd_align(heads * NC * DV * DK * 2));
    float* gq = reinterpret_cast<float*>(base + 2 * bwd_align(heads * NC * DV * DK * 2) + bwd_align(heads * DV * DK * 4));
    // forward state pass (snapshots and final memory), then the same walk backwards on (q, dO)
    ChunkArgs f{a.q, a.k, a.v, a.gate, nullptr, a.s0, nullptr, sfin, a.B, a.H, a.T, DK, DV, C, fwd};
    ChunkArgs r{a.q, a.q, a.dout, a.gate, nullptr, a.ds_out, nullptr, a.ds0, a.B, a.H, a.T, DK, DV, C, rev};
    hipError_t err = hipErrorInvalidValue;
    switch (state_value_tiles(heads, DV, DK)) {
        case 8:
            if constexpr (DV >= 128) {
                err = launch_state<C, DK, 8, GK>(f, NC, stream);
                if (err == hipSuccess) err = launch_state<C, DK, 8, GK, true>(r, NC, stream);
            }
            break;
        case 4:
            if constexpr (DV >= 64) {
                err = launch_state<C, DK, 4, GK>(f, NC, stream);
                if (err == hipSuccess) err = launch_state<C, DK, 4, GK, true>(r, NC, stream);
            }
            break;
        case 2:
            if constexpr (DV >= 32) {
                err = launch_state<C, DK, 2, GK>(f, NC, stream);
                if (err == hipSuccess) err = launch_state<C, DK, 2, GK, true>(r, NC, stream);
            }
            break;
        default:
            err = launch_state<C, DK, 1, GK>(f, NC, stream);
            if (err == hipSuccess) err = launch_state<C, DK, 1, GK, true>(r, NC, stream);
            break;
    }
    if (err != hipSuccess) return err;
    if (NC > 0) {
        GradParams p{};
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
        p.gq = gq;
        p.H = a.H;
        p.T = a.T;
        p.NC = NC;
        p.items = static_cast<int>(heads * NC);
        // persistent: as many workgroups as fit on the chip at once (one per CU at d = 128,
        // where the LDS allows one)
        int dev = 0, cus = 256, per_cu = 1;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, grad_kernel<C, DK, DV, GK>, 512, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        const int64_t slots = static_cast<int64_t>(cus) * per_cu;
        const int grid = p.items < slots ? p.items : static_cast<int>(slots);
        hipLaunchKernelGGL((grad_kernel<C, DK, DV, GK>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream, p);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if constexpr (GK == kGateScalar) {
        if (a.T == 0) return hipSuccess;
        hipLaunchKernelGGL((gate_grad_kernel<true>), dim3(static_cast<unsigned>(heads)), dim3(256), 0, stream, gq,
                           a.ds_out, sfin, a.dgate, a.T, DV * DK);
    } else {
        if (a.T > 0) {
            hipLaunchKernelGGL((gate_grad_kernel<false>), dim3(static_cast<unsigned>(heads)), dim3(256), 0, stream,
                               gq, a.ds_out, sfin, a.dgate, a.T, DV * DK);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
        hipLaunchKernelGGL(gate_head_sum_kernel, dim3(static_cast<unsigned>((a.H + 255) / 256)), dim3(256), 0, stream,
                           gq, a.dgate, a.B, a.H, a.T);
    }
    return hipGetLastError();
}

template <int C, int DK, int GK>
hipError_t launch_backward_dk(const BwdArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_backward_dv<C, DK, 16, GK>(a, stream);
        case 32: return launch_backward_dv<C, DK, 32, GK>(a, stream);
        case 64: return launch_backward_dv<C, DK, 64, GK>(a, stream);
        case 128: return launch_backward_dv<C, DK, 128, GK>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int C, int GK>
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_backward_dk<C, 16, GK>(a, stream);
        case 32: return launch_backward_dk<C, 32, GK>(a, stream);
        case 64: return launch_backward_dk<C, 64, GK>(a, stream);
        case 128: return launch_backward_dk<C, 128, GK>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
