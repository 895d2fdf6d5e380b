// Gradient pass of the gated delta rule's backward at chunk 64 (bf16 storage): every chunk's
// input gradients from the records of the forward single pass (the memory S entering the
// chunk, the pseudo-values U and R = V - diag(e^G) K S^T) and of the reverse pass (the
// gradient dS' of the memory leaving the chunk, dU, and dR, which is dV itself).
//
// Method: reverse-mode differentiation of the chunk of the gated delta rule ("Scrivere meglio
// nella memoria", sections "Correggere: la delta rule" and "Unire oblio e correzione: Gated
// DeltaNet") in its chunkwise form (RetNet page, Fig. 16.5). Per chunk, with Gamma_ij =
// e^(G_i - G_j), g = e^G, w = e^(G_last - G), A = strictly_lower(diag(beta) (K K^T . Gamma)),
// T = (I + A)^-1, T_U = T diag(beta), the forward is
//   Y = K S^T,  R = V - diag(g) Y,  U = T_U R,  O = diag(g) Q S^T + P U  (P = (Q K^T . Gamma), j <= i)
//   S_out = e^(G_last) S + U^T diag(w) K
// and, with dPG = (dO U^T) . Gamma (j <= i), dT = (dU R^T) diag(beta), dA = strictly_lower(-T^T dT T^T)
// and M = dA . (beta_i Gamma_ij) made symmetric (M + M^T):
//   dQ = diag(g) dO S + dPG K
//   dK = dPG^T Q + (M + M^T) K - diag(g) dR S + diag(w) U dS'
//   dbeta_j = sum_i (dU R^T)_ij T_ij + sum_l dA_jl (K K^T . Gamma)_jl
//   dG_i (natural log) = g_i (dO S)_i . q_i - g_i (dR S)_i . k_i + the Gamma terms of P and A
//          (row sums minus column sums of dP . P and dA . A) - w_i dw_i,
//   dG_last += sum_j w_j dw_j + e^(G_last) <dS', S>,   dw_j = (U dS')_j . k_j
// and d log alpha_t = sum_{i >= t} dG_i within the chunk.
//
// One workgroup of eight waves per chunk (persistent over the chunks):
//   stage    q, k, dO and the records U, dU, R as swizzled bf16 rows (16-byte loads, rows past
//            the sequence's end zeroed), T, gate tables;
//   phase 1  the ten lower 16 x 16 tiles of P, dP, dU R^T on bf16 MFMA: dPG to LDS (bf16), dT
//            to LDS (transposed, a bf16 hi + lo pair), and the Gamma terms of dG and the first
//            term of dbeta by row and column sums;
//   phase 2  dR is staged over dU; X = T^T dT, then the lower tiles of X T^T, on bf16 MFMA with
//            dT and X as hi + lo pairs (T is exact in bf16): dA, M (bf16, both triangles), with
//            K K^T the A terms of dG and dbeta;
//   phase 3  S and dS' over the rows' space; wave w takes token tile w % 4 and half of the key
//            tiles: dQ^T and dK^T tiles (keys along lane groups, so that each lane stores four
//            consecutive keys of one token), S, dS', Q and K by transposed LDS reads;
//   finish   one wave turns dG into d log alpha by a reverse scan and stores it with dbeta.
#pragma once

#include "chunk_delta_sp.hpp"

namespace glr {
namespace ck {

// Arguments of the gated delta rule's backward kernels (this pass and the chunk 16 / 32 ones).
struct GdBwdParams {
    const u16* q;          // [BH][T][DK]
    const u16* k;          // [BH][T][DK]
    const u16* v;          // [BH][T][DV]
    const float* alpha;    // log alpha [BH][T]
    const float* beta;     // [BH][T]
    const float* s0;       // [BH][DV][DK] or null
    const u16* dout;       // [BH][T][DV]
    const float* ds_out;   // [BH][DV][DK] or null
    u16* dq;               // [BH][T][DK]
    u16* dk;               // [BH][T][DK]
    u16* dv;               // [BH][T][DV]
    float* dalpha;         // [BH][T]
    float* dbeta;          // [BH][T]
    float* ds0;            // [BH][DV][DK] or null
    // workspace (per chunk, chunk c of sequence bh at bh * NC + c)
    const u16* tu;         // [C][C] T_U
    const float* g;        // [C] cumulative log2-gates
    const u16* tfull;      // [C][C] T
    u16* qtT;              // [DK][C] Qt^T
    u16* mp;               // [DK][DK] Mp
    u16* mpT;              // [DK][DK] Mp^T
    u16* nn;               // [DV][DK] N
    u16* sin;              // [DV][DK] memory entering the chunk
    u16* dso;              // [DV][DK] gradient of the memory leaving the chunk
    float* scratch;        // [workgroups][scratch floats]
    // records of the single passes (chunk 64): U, R = V - diag(e^G) K S_in^T and dU per
    // chunk, [BH * NC][C][DV] bf16
    const u16* rec_u;
    const u16* rec_r;
    const u16* rec_du;
    int T, NC, chunks;
};

template <int DK, int DV>
struct GdGradLayout {
    static constexpr int C = 64;
    using TK = SwzTile<DK>;                 // q, k rows [C][DK]; S, dS' rows [DV][DK]
    using TV = SwzTile<DV>;                 // dO, U, dU, R and dR rows [C][DV]
    static constexpr int RS = C + 8;        // bf16 rows of dPG, M, T, dT^T and X
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int KBYTES = al(C * TK::STRIDE * 2);     // one [C][DK] tile
    static constexpr int SBYTES = al(DV * TK::STRIDE * 2);    // one [DV][DK] tile
    static constexpr int RB = al(C * TV::STRIDE * 2);         // one [C][DV] tile
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + KBYTES;
    static constexpr int oP = oK + KBYTES;
    static constexpr int oM = oP + al(C * RS * 2);
    // region A: the rows of dO, U, dU and R (slots 0-3; dR takes slot 2 once dU is done), then
    // S and dS'
    static constexpr int oA = oM + al(C * RS * 2);
    static constexpr int AB = 4 * RB > 2 * SBYTES ? 4 * RB : 2 * SBYTES;
    // region B: T, then dT^T as a bf16 hi + lo pair (which X then replaces)
    static constexpr int oT = oA + AB;
    static constexpr int oH = oT + al(C * RS * 2);
    static constexpr int oL = oH + al(C * RS * 2);
    static constexpr int oSum = oL + al(C * RS * 2);
    // per-token sums: dG, dbeta, dw; tables: G (log2), e^G, e^(G_last - G), beta; then <dS', S>
    static constexpr int SG = 0, SB = C, SW = 2 * C, TG = 3 * C, TEG = 4 * C, TW = 5 * C, TBE = 6 * C, STR = 7 * C;
    static constexpr int bytes = oSum + al((7 * C + 4) * 4);
    static_assert(bytes <= 160 * 1024, "LDS budget of the gated delta gradient pass exceeded");
};

inline int gd_grads_workgroups(int64_t chunks) { return static_cast<int>(chunks < kCUs ? chunks : kCUs); }

// Lane (r16, g) of a 16 x 16 tile holds D[4g + e][r16]: sums over the tile's columns (per row
// 4g + e, in every lane of the row group) and over its rows (per column r16, in every lane
// of the column).
__device__ __forceinline__ f32x4 tile_row_sums(f32x4 x) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = row16_sum(x[e]);
    return r;
}
__device__ __forceinline__ float tile_col_sum(f32x4 x) { return cross_row_sum(x[0] + x[1] + x[2] + x[3]); }

template <int DK, int DV>
__global__ __launch_bounds__(512)
void gd_grads_kernel(GdBwdParams p) {
    using Lay = GdGradLayout<DK, DV>;
    using TK = typename Lay::TK;
    using TV = typename Lay::TV;
    constexpr int C = 64, CT = 4, JB = 2, KB = DK / 32, VB = DV / 32, KTL = DK / 16, KW = KTL / 2;
    constexpr int NT = 512, RS = Lay::RS;
    static_assert(DK % 32 == 0 && DV % 32 == 0, "d_k and d_v in 32-channel blocks");

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    u16* const sQ = reinterpret_cast<u16*>(smem + Lay::oQ);
    u16* const sK = reinterpret_cast<u16*>(smem + Lay::oK);
    u16* const sPG = reinterpret_cast<u16*>(smem + Lay::oP);
    u16* const sM = reinterpret_cast<u16*>(smem + Lay::oM);
    auto slot = [&](int i) { return reinterpret_cast<u16*>(smem + Lay::oA + i * Lay::RB); };
    u16* const sdO = slot(0);
    u16* const sU = slot(1);
    u16* const sdU = slot(2);   // then dR
    u16* const sR = slot(3);
    u16* const sS = reinterpret_cast<u16*>(smem + Lay::oA);
    u16* const sdS = reinterpret_cast<u16*>(smem + Lay::oA + Lay::SBYTES);
    u16* const sT = reinterpret_cast<u16*>(smem + Lay::oT);
    u16* const sHi = reinterpret_cast<u16*>(smem + Lay::oH);   // dT^T, then X: bf16 hi part
    u16* const sLo = reinterpret_cast<u16*>(smem + Lay::oL);   // and the residual
    float* const sm = reinterpret_cast<float*>(smem + Lay::oSum);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    // the lower tiles (it >= jt) in row order
    auto tile_of = [](int pr, int& it, int& jt) {
        it = 0;
        jt = pr;
        while (jt > it) {
            jt -= it + 1;
            ++it;
        }
    };
    // MFMA operands: from a bf16 row, slots 32b + 4g + e and 32b + 16 + 4g + e; from a row of a
    // swizzled tile; and transposed (lane (r16, g) gets X[32b + 4g + e][n0 + r16], then + 16)
    auto row_op = [&](const u16* row, int b) { return join8(ld4(row + 32 * b + 4 * g), ld4(row + 32 * b + 16 + 4 * g)); };
    auto row_k = [&](const u16* X, int r, int b) {
        return join8(ld4(X + TK::off(r, 32 * b + 4 * g)), ld4(X + TK::off(r, 32 * b + 16 + 4 * g)));
    };
    auto row_v = [&](const u16* X, int r, int b) {
        return join8(ld4(X + TV::off(r, 32 * b + 4 * g)), ld4(X + TV::off(r, 32 * b + 16 + 4 * g)));
    };
    auto col_k = [&](const u16* X, int b, int n0) {
        return join8(tr_op_s<DK>(X, 32 * b, n0, r16, g), tr_op_s<DK>(X, 32 * b + 16, n0, r16, g));
    };
    auto bfv = [](u16 x) { return bf16_bits_to_f32(x); };
    // 16-byte pieces of [rows][W] tiles: piece i of this thread is idx = tid + NT i (every
    // thread the same count; all of a stage's loads are issued before its LDS writes, so that
    // one wait covers them)
    constexpr int PR = C * DV / 8, PR_PER = (PR + NT - 1) / NT;      // [C][DV] rows
    constexpr int PK = C * DK / 8, PK_PER = (PK + NT - 1) / NT;      // [C][DK] rows
    constexpr int PS = DV * DK / 8, PS_PER = (PS + NT - 1) / NT;     // [DV][DK]
    constexpr int PT = C * C / 8, PT_PER = (PT + NT - 1) / NT;       // [C][C]
    // rows [C][DV] of a token-major tensor (or record): loads (rows past the sequence's end read
    // its last row when `mask`) and their LDS writes (those rows zeroed)
    auto load_rows = [&](u16x8 (&r)[PR_PER], const u16* src, int n, bool mask) {
#pragma unroll
        for (int i = 0; i < PR_PER; ++i) {
            const int idx = tid + NT * i;
            const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            const int jr = (mask && j >= n) ? n - 1 : j;
            r[i] = idx < PR ? *reinterpret_cast<const u16x8*>(src + static_cast<int64_t>(jr) * DV + col) : z8;
        }
    };
    auto write_rows = [&](u16* dst, const u16x8 (&r)[PR_PER], int n, bool mask) {
#pragma unroll
        for (int i = 0; i < PR_PER; ++i) {
            const int idx = tid + NT * i;
            const int j = idx / (DV / 8), col = (idx % (DV / 8)) * 8;
            if (idx < PR) *reinterpret_cast<u16x8*>(dst + TV::off(j, col)) = (mask && j >= n) ? z8 : r[i];
        }
    };

    for (int chunk = blockIdx.x; chunk < p.chunks; chunk += gridDim.x) {
        const int bh = chunk / p.NC, c = chunk % p.NC;
        const int t0 = c * C, n = (p.T - t0 < C) ? (p.T - t0) : C;
        const int64_t tok0 = static_cast<int64_t>(bh) * p.T + t0;
        const int64_t rec0 = static_cast<int64_t>(chunk) * C;   // records' token rows

        // ---------------------------------------------------------------- stage
        // q, k, dO (rows past the sequence's end zeroed, their loads reading its last row) and
        // the records U, dU, R; T; zeroed dT, dPG and M; the gate tables
        {
            u16x8 rq[PK_PER], rk[PK_PER], ro[PR_PER], ru[PR_PER], rdu[PR_PER], rr[PR_PER], rt[PT_PER];
#pragma unroll
            for (int i = 0; i < PK_PER; ++i) {
                const int idx = tid + NT * i;
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                const int64_t at = (tok0 + (j < n ? j : n - 1)) * DK + col;
                rq[i] = idx < PK ? *reinterpret_cast<const u16x8*>(p.q + at) : z8;
                rk[i] = idx < PK ? *reinterpret_cast<const u16x8*>(p.k + at) : z8;
            }
            load_rows(ro, p.dout + tok0 * DV, n, true);
            load_rows(ru, p.rec_u + rec0 * DV, n, false);
            load_rows(rdu, p.rec_du + rec0 * DV, n, false);
            load_rows(rr, p.rec_r + rec0 * DV, n, false);
            const u16* Tg = p.tfull + static_cast<int64_t>(chunk) * C * C;
#pragma unroll
            for (int i = 0; i < PT_PER; ++i) {
                const int idx = tid + NT * i;
                rt[i] = idx < PT ? *reinterpret_cast<const u16x8*>(Tg + idx * 8) : z8;
            }
#pragma unroll
            for (int i = 0; i < PK_PER; ++i) {
                const int idx = tid + NT * i;
                const int j = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                if (idx < PK) {
                    *reinterpret_cast<u16x8*>(sQ + TK::off(j, col)) = j < n ? rq[i] : z8;
                    *reinterpret_cast<u16x8*>(sK + TK::off(j, col)) = j < n ? rk[i] : z8;
                }
            }
            write_rows(sdO, ro, n, true);
            write_rows(sU, ru, n, false);
            write_rows(sdU, rdu, n, false);
            write_rows(sR, rr, n, false);
#pragma unroll
            for (int i = 0; i < PT_PER; ++i) {
                const int idx = tid + NT * i;
                if (idx < PT) *reinterpret_cast<u16x8*>(sT + (idx / (C / 8)) * RS + (idx % (C / 8)) * 8) = rt[i];
            }
        }
        for (int idx = tid; idx < C * RS / 2; idx += NT) {
            reinterpret_cast<unsigned*>(sPG)[idx] = 0u;
            reinterpret_cast<unsigned*>(sM)[idx] = 0u;
            reinterpret_cast<unsigned*>(sHi)[idx] = 0u;
            reinterpret_cast<unsigned*>(sLo)[idx] = 0u;
        }
        if (tid < C) {
            const float G = p.g[rec0 + tid];
            const float Gl = p.g[rec0 + C - 1];
            sm[Lay::SG + tid] = 0.f;
            sm[Lay::SB + tid] = 0.f;
            sm[Lay::SW + tid] = 0.f;
            sm[Lay::TG + tid] = G;
            sm[Lay::TEG + tid] = ex2(G);
            sm[Lay::TW + tid] = ex2(Gl - G);
            sm[Lay::TBE + tid] = tid < n ? p.beta[tok0 + tid] : 0.f;
        }
        if (tid == 0) sm[Lay::STR] = 0.f;
        __syncthreads();

        // ---------------------------------------------------------------- phase 1
        // dR's loads go out now and land over dU after this phase
        u16x8 rdr[PR_PER];
        load_rows(rdr, p.dv + tok0 * DV, n, true);
        for (int pr = w; pr < CT * (CT + 1) / 2; pr += 8) {
            int it, jt;
            tile_of(pr, it, jt);
            const int ia = 16 * it + r16, ja = 16 * jt + r16;   // operand rows of this lane
            f32x4 s = zf4(), dp = zf4(), dtu = zf4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s = mfma_16x16x32(row_k(sQ, ia, kb), row_k(sK, ja, kb), s);
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
                dp = mfma_16x16x32(row_v(sdO, ia, vb), row_v(sU, ja, vb), dp);
                dtu = mfma_16x16x32(row_v(sdU, ia, vb), row_v(sR, ja, vb), dtu);
            }
            // element (i, j) = (16it + 4g + e, 16jt + r16)
            const int j = 16 * jt + r16;
            const float Gj = sm[Lay::TG + j], bj = sm[Lay::TBE + j];
            f32x4 dpp, gdb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * g + e;
                const bool in = j <= i;
                const float gam = in ? ex2(sm[Lay::TG + i] - Gj) : 0.f;
                const float pg = dp[e] * gam;
                dpp[e] = pg * s[e];                      // dP . P
                sPG[i * RS + j] = __builtin_bit_cast(u16, static_cast<__bf16>(pg));
                const float dt = in ? dtu[e] : 0.f;
                gdb[e] = dt * bfv(sT[i * RS + j]);       // dbeta_j: (dU R^T)_ij T_ij
                // dT^T[j][i] as hi + lo
                const __bf16 h = static_cast<__bf16>(dt * bj);
                sHi[j * RS + i] = __builtin_bit_cast(u16, h);
                sLo[j * RS + i] = __builtin_bit_cast(u16, static_cast<__bf16>(dt * bj - static_cast<float>(h)));
            }
            const f32x4 rs = tile_row_sums(dpp);
            const float cs = tile_col_sum(dpp), cb = tile_col_sum(gdb);
            if (r16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) atomicAdd(&sm[Lay::SG + 16 * it + 4 * g + e], rs[e]);
            }
            if (g == 0) {
                atomicAdd(&sm[Lay::SG + j], -cs);
                atomicAdd(&sm[Lay::SB + j], cb);
            }
        }
        __syncthreads();

        // ---------------------------------------------------------------- phase 2
        // dR over dU (read with dO and U once phase 2 is done); the loads of S and dS' go out
        // now and land over the rows after phase 2
        write_rows(sdU, rdr, n, true);
        const u16* Sg = p.sin + static_cast<int64_t>(chunk) * DV * DK;
        const u16* dSg = p.dso + static_cast<int64_t>(chunk) * DV * DK;
        u16x8 rs_[PS_PER], rd_[PS_PER];
#pragma unroll
        for (int i = 0; i < PS_PER; ++i) {
            const int idx = tid + NT * i;
            rs_[i] = idx < PS ? *reinterpret_cast<const u16x8*>(Sg + idx * 8) : z8;
            rd_[i] = idx < PS ? *reinterpret_cast<const u16x8*>(dSg + idx * 8) : z8;
        }
        // X = T^T dT: X[i][l] = sum_{m >= max(i, l)} T[m][i] dT[m][l] on bf16 MFMA (T is exact in
        // bf16; dT as hi + lo), T^T by transposed reads, dT^T by rows; held until every wave has
        // read dT^T, then written over it as hi + lo rows
        f32x4 xt[2];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int t = w + 8 * q2;
            const int it = t / CT, lt = t % CT;
            const int m_lo = 16 * (it > lt ? it : lt);
            f32x4 acc = zf4();
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                if (32 * b + 31 < m_lo) continue;
                const bf16x8 ta = join8(tr_op<RS>(sT, 32 * b, 16 * it, r16, g), tr_op<RS>(sT, 32 * b + 16, 16 * it, r16, g));
                acc = mfma_16x16x32(ta, row_op(sHi + (16 * lt + r16) * RS, b), acc);
                acc = mfma_16x16x32(ta, row_op(sLo + (16 * lt + r16) * RS, b), acc);
            }
            xt[q2] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int t = w + 8 * q2;
            const int it = t / CT, lt = t % CT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int at = (16 * it + 4 * g + e) * RS + 16 * lt + r16;
                const __bf16 h = static_cast<__bf16>(xt[q2][e]);
                sHi[at] = __builtin_bit_cast(u16, h);
                sLo[at] = __builtin_bit_cast(u16, static_cast<__bf16>(xt[q2][e] - static_cast<float>(h)));
            }
        }
        __syncthreads();
        // dA = strictly_lower(-X T^T): (X T^T)[i][j] = sum_{l <= j} X[i][l] T[j][l]
        for (int pr = w; pr < CT * (CT + 1) / 2; pr += 8) {
            int it, jt;
            tile_of(pr, it, jt);
            const int ia = 16 * it + r16, ja = 16 * jt + r16;
            f32x4 y = zf4(), kk = zf4();
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                if (32 * b > 16 * jt + 15) continue;
                const bf16x8 tb = row_op(sT + ja * RS, b);
                y = mfma_16x16x32(row_op(sHi + ia * RS, b), tb, y);
                y = mfma_16x16x32(row_op(sLo + ia * RS, b), tb, y);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) kk = mfma_16x16x32(row_k(sK, ia, kb), row_k(sK, ja, kb), kk);
            const int j = 16 * jt + r16;
            const float Gj = sm[Lay::TG + j];
            f32x4 daa, dkg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * it + 4 * g + e;
                const bool in = j < i;
                const float bi = sm[Lay::TBE + i];
                const float gam = in ? ex2(sm[Lay::TG + i] - Gj) : 0.f;
                const float da = in ? -y[e] : 0.f;
                const float kg = kk[e] * gam;            // (K K^T . Gamma)_ij
                dkg[e] = da * kg;                         // dbeta_i
                daa[e] = dkg[e] * bi;                     // dA . A
                if (in) {
                    const u16 mv = __builtin_bit_cast(u16, static_cast<__bf16>(da * bi * gam));
                    sM[i * RS + j] = mv;
                    sM[j * RS + i] = mv;
                }
            }
            const f32x4 rs = tile_row_sums(daa), rb = tile_row_sums(dkg);
            const float cs = tile_col_sum(daa);
            if (r16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    atomicAdd(&sm[Lay::SG + 16 * it + 4 * g + e], rs[e]);
                    atomicAdd(&sm[Lay::SB + 16 * it + 4 * g + e], rb[e]);
                }
            }
            if (g == 0) atomicAdd(&sm[Lay::SG + j], -cs);
        }
        __syncthreads();

        // ---------------------------------------------------------------- phase 3
        // wave w's rows (token tile w % 4) of dO, U and dR into registers; then S and dS' over
        // their space, with <dS', S> on the way
        const int it3 = w % CT;
        const int tok = 16 * it3 + r16;
        bf16x8 bo[VB], bu[VB], br[VB];
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
            bo[vb] = row_v(sdO, tok, vb);
            bu[vb] = row_v(sU, tok, vb);
            br[vb] = row_v(sdU, tok, vb);
        }
        __syncthreads();
        {
            float tr = 0.f;
#pragma unroll
            for (int i = 0; i < PS_PER; ++i) {
                const int idx = tid + NT * i;
                const int v = idx / (DK / 8), col = (idx % (DK / 8)) * 8;
                if (idx < PS) {
                    *reinterpret_cast<u16x8*>(sS + TK::off(v, col)) = rs_[i];
                    *reinterpret_cast<u16x8*>(sdS + TK::off(v, col)) = rd_[i];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) tr += bfv(rs_[i][e]) * bfv(rd_[i][e]);
            }
            tr = wave_sum(tr);
            if (lane == 0) atomicAdd(&sm[Lay::STR], tr);
        }
        __syncthreads();
        {
            // wave w: token tile it3, key tiles KW kh .. KW kh + KW - 1 (this lane's token: tok)
            const int kh = w / CT;
            const bool live = tok < n;
            const float gi = sm[Lay::TEG + tok], wi = sm[Lay::TW + tok];
            bf16x8 bp[JB], bpt[JB], bm[JB];
#pragma unroll
            for (int b = 0; b < JB; ++b) {
                bp[b] = row_op(sPG + tok * RS, b);                         // dPG[tok][j]
                bm[b] = row_op(sM + tok * RS, b);                          // M[tok][j] (symmetric)
                bpt[b] = join8(tr_op<RS>(sPG, 32 * b, 16 * it3, r16, g),   // dPG[i][tok]
                               tr_op<RS>(sPG, 32 * b + 16, 16 * it3, r16, g));
            }
            float dgq = 0.f, dgk = 0.f, dwk = 0.f;
#pragma unroll 2
            for (int kk2 = 0; kk2 < KW; ++kk2) {
                const int kt = kh * KW + kk2;
                // keys 16kt + 4g + e of this lane: q and k of its token
                const f32x4 qk = up4(ld4(sQ + TK::off(tok, 16 * kt + 4 * g)));
                const f32x4 kq = up4(ld4(sK + TK::off(tok, 16 * kt + 4 * g)));
                // dQ^T tile: g_i (dO S)^T + (dPG K)^T; dK^T tile: -g_j (dR S)^T + w_j (U dS')^T
                // + (dPG^T Q)^T + ((M + M^T) K)^T
                f32x4 a1 = zf4(), za = zf4(), zb = zf4();
#pragma unroll
                for (int vb = 0; vb < VB; ++vb) {
                    const bf16x8 st = col_k(sS, vb, 16 * kt);     // S[v][key]
                    a1 = mfma_16x16x32(st, bo[vb], a1);
                    za = mfma_16x16x32(st, br[vb], za);
                    zb = mfma_16x16x32(col_k(sdS, vb, 16 * kt), bu[vb], zb);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dgq += a1[e] * qk[e];
                    dgk += za[e] * kq[e];
                    dwk += zb[e] * kq[e];
                }
                f32x4 dq = a1 * gi;
                f32x4 dk = za * (-gi) + zb * wi;
#pragma unroll
                for (int b = 0; b < JB; ++b) {
                    const bf16x8 kc = col_k(sK, b, 16 * kt);      // K[j][key]
                    if (32 * b <= 16 * it3 + 15) dq = mfma_16x16x32(kc, bp[b], dq);
                    if (32 * b + 31 >= 16 * it3) dk = mfma_16x16x32(col_k(sQ, b, 16 * kt), bpt[b], dk);
                    dk = mfma_16x16x32(kc, bm[b], dk);
                }
                if (live) {
                    st4(p.dq + (tok0 + tok) * DK + 16 * kt + 4 * g, cvt4(dq));
                    st4(p.dk + (tok0 + tok) * DK + 16 * kt + 4 * g, cvt4(dk));
                }
            }
            dgq = cross_row_sum(dgq);
            dgk = cross_row_sum(dgk);
            dwk = cross_row_sum(dwk);
            if (g == 0) {
                atomicAdd(&sm[Lay::SG + tok], gi * (dgq - dgk));
                atomicAdd(&sm[Lay::SW + tok], dwk);
            }
        }
        __syncthreads();

        // ---------------------------------------------------------------- finish
        if (w == 0) {
            const float wl = sm[Lay::TW + lane], dw = sm[Lay::SW + lane];
            float x = sm[Lay::SG + lane] - wl * dw;
            const float wsum = wave_sum(wl * dw);
            if (lane == C - 1) x += wsum + ex2(sm[Lay::TG + C - 1]) * sm[Lay::STR];
            // d log alpha_t = sum_{i >= t} dG_i: reverse inclusive scan over the 64 lanes
            float y = x;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float t = __shfl_down(y, off, 64);
                if (lane + off < 64) y += t;
            }
            if (lane < n) {
                p.dalpha[tok0 + lane] = y;
                p.dbeta[tok0 + lane] = sm[Lay::SB + lane];
            }
        }
        __syncthreads();
    }
}

}  // namespace ck
}  // namespace glr
