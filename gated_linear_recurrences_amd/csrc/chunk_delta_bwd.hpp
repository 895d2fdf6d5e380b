// Backward of the gated delta rule, bf16 storage: the gradients of q, k, v, log alpha, beta and
// the initial memory for L = <dO, o> + <dS_T, S_T>.
//
// Method: reverse-mode differentiation of the chunkwise form of the gated delta rule ("Scrivere
// meglio nella memoria", sections "Correggere: la delta rule" for the UT form and "Unire oblio
// e correzione: Gated DeltaNet"; the chunkwise form of the RetNet page, Fig. 16.5). Per chunk of
// n tokens with cumulative log-gates G, g = e^G, w = e^(G_last - G), Gamma_ij = e^(G_i - G_j),
// A = strictly_lower(diag(beta) (K K^T . Gamma)), T = (I + A)^-1, T_U = T diag(beta):
//   W = T_U diag(g) K,  U0 = T_U V,  P = (Q K^T . Gamma) masked (j <= i),
// the chunk is a linear map of the memory S entering it:
//   O     = Qt S^T + P U0,                  Qt = diag(g) Q - P W
//   S_out = S (e^(G_last) I + Mp) + N,      Mp = -W^T diag(w) K,  N = U0^T diag(w) K
// so the memory's gradient runs back through the chunks as
//   dS_in = e^(G_last) dS_out + dS_out Mp^T + dO^T Qt,
// and with the memory entering and the gradient leaving every chunk known, each chunk's input
// gradients are independent (the products are listed in grads_kernel).
//
// At chunk 64 with d_k >= 32 the call takes the single-pass form instead (launch below): the
// prep, the forward single pass recording S_in, U and R per chunk, the same pass in reverse
// for dS', dU, dV and ds0 (chunk_delta_sp.hpp), and gd_grads_kernel (chunk_delta_grads.hpp;
// d_v = 16 keeps grads_kernel). Chunks 16 and 32 take the linear-map form here.
//
// Linear-map kernels, in order on the stream:
//   prep     delta_tfac_kernel (G, T_U, and T itself), all chunks in parallel;
//   maps     maps_kernel: W, U0, P, then Qt^T, Mp, Mp^T and N per chunk (bf16, workspace);
//   forward  fwd_chain_kernel: per (sequence, 16 value rows), the memory entering every chunk
//            (bf16), S^T <- e^(G_last) S^T + Mp^T S^T + N^T;
//   reverse  bwd_chain_kernel: per (sequence, 16 value rows), the gradient leaving every chunk
//            (bf16) and ds0, dS^T <- e^(G_last) dS^T + Mp dS^T + Qt^T dO;
//   grads    grads_kernel: dq, dk, dv, dbeta and d log alpha per chunk.
// The chains hold S^T (dS^T) for 16 value rows in fp32 MFMA accumulators; with 16x16x16 bf16
// products an accumulator tile is the next product's B operand as it stands. maps and grads
// run their products with gemm_lds (16 x 16 output tiles on fp32 MFMA, operands read through
// loader functions and staged slice by slice in LDS) over a per-workgroup fp32 scratch in
// global memory: persistent workgroups take the chunks in turn.
#pragma once

#include "chunk_delta_grads.hpp"

namespace glr {
namespace ck {

// fp32 scratch of one maps / grads workgroup (floats)
template <int C, int DK, int DV>
struct GdScratch {
    static constexpr int CK = C * DK, CV = C * DV, CC = C * C, KK = DK * DK;
    static constexpr int W = 0, U0 = W + CK, P = U0 + CV, DQT = P + CC, DM = DQT + CK, DU0 = DM + KK, DP = DU0 + CV,
                         DW = DP + CC, DKX = DW + CK, TDW = DKX + CK, TDU = TDW + CK, DT = TDU + CV, Z = DT + CC,
                         DA = Z + CC, KG = DA + CC, DQ2 = KG + CC;
    static constexpr int floats = DQ2 + CK;
};

inline int gd_bwd_workgroups(int64_t chunks) { return static_cast<int>(chunks < 512 ? chunks : 512); }

inline size_t gd_bwd_ws_bytes(int64_t chunks, int C, int dk, int dv) {
    const int64_t CK = static_cast<int64_t>(C) * dk, CV = static_cast<int64_t>(C) * dv;
    const int64_t CC = static_cast<int64_t>(C) * C, KK = static_cast<int64_t>(dk) * dk;
    const int64_t VK = static_cast<int64_t>(dv) * dk;
    const int64_t scr = 6 * CK + 3 * CV + 6 * CC + KK;   // GdScratch<C, DK, DV>::floats
    return delta_ws_align(chunks * CC * 2) + delta_ws_align(chunks * C * 4) + delta_ws_align(chunks * CC * 2) +
           delta_ws_align(chunks * CK * 2) + 2 * delta_ws_align(chunks * KK * 2) + 3 * delta_ws_align(chunks * VK * 2) +
           3 * delta_ws_align(chunks * CV * 2) + delta_ws_align(gd_bwd_workgroups(chunks) * scr * 4);
}

__device__ __forceinline__ float bf(u16 x) { return bf16_bits_to_f32(x); }
// A scratch value written by another wave of the workgroup before the last barrier: read at
// device scope, past the CU's vector cache (which may still hold the previous chunk's line).
__device__ __forceinline__ float scr(const float* x) { return __hip_atomic_load(x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u16 to_bf(float x) { return __builtin_bit_cast(u16, static_cast<__bf16>(x)); }

// out(m, n) <- epi(m, n, sum_k x(m, k) y(k, n)) for an M x N output (multiples of 16) and a
// reduction over K (a multiple of 16), on fp32 MFMA 16x16x4 (lane (r, g) supplies x(m0 + r, k)
// and y(k, n0 + r) for k = k0 + g and receives rows m0 + 4g + e of column n0 + r). The
// reduction runs in slices of KS: every slice of x and y is first copied by the whole
// workgroup into LDS (each element read once, neighbouring threads on neighbouring elements),
// then each wave takes its 16 x 16 output tiles from LDS. Row strides of the staged slices
// put the 16 rows x 4 reduction slots of one operand read in 64 distinct banks.
constexpr int kGemmMax = 128;                                   // largest M or N
constexpr int kSliceMax = 64;                                   // largest reduction slice
constexpr int gemm_sy(int n) { return n + ((16 - n) % 64 + 64) % 64; }
constexpr int kSxFloats = kGemmMax * (kSliceMax + 4);
constexpr int kSyFloats = kSliceMax * gemm_sy(kGemmMax);

template <int M, int N, int K, typename FX, typename FY, typename FE>
__device__ __forceinline__ void gemm_lds(float* sx, float* sy, FX x, FY y, FE epi) {
    static_assert(M % 16 == 0 && N % 16 == 0 && K % 16 == 0 && M <= kGemmMax && N <= kGemmMax, "gemm shape");
    constexpr int KS = K % 64 == 0 ? 64 : (K % 32 == 0 ? 32 : 16);
    constexpr int SX = KS + 4, SY = gemm_sy(N);
    constexpr int TN = N / 16, TILES = (M / 16) * TN, PER = (TILES + 3) / 4;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    f32x4 acc[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) acc[q] = zf4();
    for (int k0 = 0; k0 < K; k0 += KS) {
        for (int idx = tid; idx < M * KS; idx += 256) sx[(idx / KS) * SX + idx % KS] = x(idx / KS, k0 + idx % KS);
        for (int idx = tid; idx < KS * N; idx += 256) sy[(idx / N) * SY + idx % N] = y(k0 + idx / N, idx % N);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int t = w + 4 * q;
            if (t < TILES) {
                const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
#pragma unroll 4
                for (int k = 0; k < KS; k += 4)
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(sx[(m0 + r) * SX + k + g], sy[(k + g) * SY + n0 + r],
                                                                  acc[q], 0, 0, 0);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int t = w + 4 * q;
        if (t < TILES) {
            const int m0 = (t / TN) * 16, n0 = (t % TN) * 16;
#pragma unroll
            for (int e = 0; e < 4; ++e) epi(m0 + 4 * g + e, n0 + r, acc[q][e]);
        }
    }
}

// ====================================================================== maps
template <int C, int DK, int DV>
__global__ __launch_bounds__(256)
void maps_kernel(GdBwdParams p) {
    using S = GdScratch<C, DK, DV>;
    float* const sc = p.scratch + static_cast<int64_t>(blockIdx.x) * S::floats;
    __shared__ float sg[C], sw[C];   // e^G, e^(G_last - G)
    __shared__ float sx[kSxFloats], sy[kSyFloats];
    for (int chunk = blockIdx.x; chunk < p.chunks; chunk += gridDim.x) {
        const int bh = chunk / p.NC, c = chunk % p.NC;
        const int t0 = c * C, n = (p.T - t0 < C) ? (p.T - t0) : C;
        const int64_t tok0 = static_cast<int64_t>(bh) * p.T + t0;
        const u16* K = p.k + tok0 * DK;
        const u16* Q = p.q + tok0 * DK;
        const u16* V = p.v + tok0 * DV;
        const float* G = p.g + static_cast<int64_t>(chunk) * C;
        const u16* TU = p.tu + static_cast<int64_t>(chunk) * C * C;
        if (threadIdx.x < C) {
            sg[threadIdx.x] = ex2(G[threadIdx.x]);
            sw[threadIdx.x] = ex2(G[C - 1] - G[threadIdx.x]);
        }
        __syncthreads();
        auto kx = [&](int j, int a) { return j < n ? bf(K[j * DK + a]) : 0.f; };
        // W = T_U diag(g) K, U0 = T_U V, P = (Q K^T . Gamma) masked
        gemm_lds<C, DK, C>(sx, sy, [&](int i, int j) { return bf(TU[i * C + j]); }, [&](int j, int a) { return sg[j] * kx(j, a); },
                  [&](int i, int a, float v) { sc[S::W + i * DK + a] = v; });
        gemm_lds<C, DV, C>(sx, sy, [&](int i, int j) { return bf(TU[i * C + j]); },
                  [&](int j, int m) { return j < n ? bf(V[j * DV + m]) : 0.f; },
                  [&](int i, int m, float v) { sc[S::U0 + i * DV + m] = v; });
        gemm_lds<C, C, DK>(sx, sy, [&](int i, int a) { return i < n ? bf(Q[i * DK + a]) : 0.f; }, [&](int a, int j) { return kx(j, a); },
                  [&](int i, int j, float v) { sc[S::P + i * C + j] = j <= i ? v * ex2(G[i] - G[j]) : 0.f; });
        __syncthreads();
        // Qt = diag(g) Q - P W (stored transposed), Mp = -W^T diag(w) K (and transposed),
        // N = U0^T diag(w) K
        u16* qtT = p.qtT + static_cast<int64_t>(chunk) * DK * C;
        u16* mp = p.mp + static_cast<int64_t>(chunk) * DK * DK;
        u16* mpT = p.mpT + static_cast<int64_t>(chunk) * DK * DK;
        u16* nn = p.nn + static_cast<int64_t>(chunk) * DV * DK;
        gemm_lds<C, DK, C>(sx, sy, [&](int i, int j) { return scr(sc + S::P + i * C + j); }, [&](int j, int a) { return scr(sc + S::W + j * DK + a); },
                  [&](int i, int a, float v) {
                      const float qv = i < n ? bf(Q[i * DK + a]) : 0.f;
                      qtT[a * C + i] = to_bf(sg[i] * qv - v);
                  });
        gemm_lds<DK, DK, C>(sx, sy, [&](int a, int j) { return scr(sc + S::W + j * DK + a); }, [&](int j, int b) { return sw[j] * kx(j, b); },
                  [&](int a, int b, float v) {
                      mp[a * DK + b] = to_bf(-v);
                      mpT[b * DK + a] = to_bf(-v);
                  });
        gemm_lds<DV, DK, C>(sx, sy, [&](int m, int j) { return scr(sc + S::U0 + j * DV + m); }, [&](int j, int b) { return sw[j] * kx(j, b); },
                  [&](int m, int b, float v) { nn[m * DK + b] = to_bf(v); });
        __syncthreads();
    }
}

// ====================================================================== chains
// One wave per (sequence, 16 value rows v0 .. v0 + 15); tiles ct of the memory (or its
// gradient) transposed: acc[ct][e] = X^T[16ct + 4g + e][v0 + r16] = X[v0 + r16][16ct + 4g + e].
template <int C, int DK, int DV>
__global__ __launch_bounds__(64)
void fwd_chain_kernel(GdBwdParams p) {
    constexpr int KT = DK / 16;
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / (DV / 16), v0 = (blockIdx.x % (DV / 16)) * 16;
    f32x4 acc[KT];
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
        acc[ct] = p.s0 ? ldf4(p.s0 + (static_cast<int64_t>(bh) * DV + v0 + r16) * DK + 16 * ct + 4 * g) : zf4();
    for (int c = 0; c < p.NC; ++c) {
        const int64_t chunk = static_cast<int64_t>(bh) * p.NC + c;
        u16* sin = p.sin + chunk * DV * DK + (v0 + r16) * DK;
        const u16* mpT = p.mpT + chunk * DK * DK;
        const u16* nn = p.nn + chunk * DV * DK + (v0 + r16) * DK;
        const float gl = ex2(p.g[chunk * C + C - 1]);
        bf16x4 xb[KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            xb[ct] = cvt4(acc[ct]);
            *reinterpret_cast<bf16x4*>(sin + 16 * ct + 4 * g) = xb[ct];
        }
        // S^T <- e^(G_last) S^T + Mp^T S^T + N^T
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            f32x4 nv = up4(*reinterpret_cast<const bf16x4*>(nn + 16 * ct + 4 * g));
            f32x4 s = acc[ct] * gl + nv;
#pragma unroll
            for (int cb = 0; cb < KT; ++cb) {
                const bf16x4 a = *reinterpret_cast<const bf16x4*>(mpT + (16 * ct + r16) * DK + 16 * cb + 4 * g);
                s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, xb[cb], s, 0, 0, 0);
            }
            acc[ct] = s;
        }
    }
}

template <int C, int DK, int DV>
__global__ __launch_bounds__(64)
void bwd_chain_kernel(GdBwdParams p) {
    constexpr int KT = DK / 16, TB = C / 16;
    const int lane = threadIdx.x, r16 = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x / (DV / 16), v0 = (blockIdx.x % (DV / 16)) * 16;
    f32x4 acc[KT];
#pragma unroll
    for (int ct = 0; ct < KT; ++ct)
        acc[ct] = p.ds_out ? ldf4(p.ds_out + (static_cast<int64_t>(bh) * DV + v0 + r16) * DK + 16 * ct + 4 * g) : zf4();
    for (int c = p.NC - 1; c >= 0; --c) {
        const int64_t chunk = static_cast<int64_t>(bh) * p.NC + c;
        const int t0 = c * C, n = (p.T - t0 < C) ? (p.T - t0) : C;
        u16* dso = p.dso + chunk * DV * DK + (v0 + r16) * DK;
        const u16* mp = p.mp + chunk * DK * DK;
        const u16* qtT = p.qtT + chunk * DK * C;
        const u16* dO = p.dout + (static_cast<int64_t>(bh) * p.T + t0) * DV + v0 + r16;
        const float gl = ex2(p.g[chunk * C + C - 1]);
        bf16x4 xb[KT], ob[TB];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            xb[ct] = cvt4(acc[ct]);
            *reinterpret_cast<bf16x4*>(dso + 16 * ct + 4 * g) = xb[ct];
        }
        // dO[t][v0 + r16] for t = 16tb + 4g + e (zero past the sequence's end)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tb + 4 * g + e;
                ob[tb][e] = __builtin_bit_cast(__bf16, t < n ? dO[static_cast<int64_t>(t) * DV] : static_cast<u16>(0));
            }
        // dS^T <- e^(G_last) dS^T + Mp dS^T + Qt^T dO
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            f32x4 s = acc[ct] * gl;
#pragma unroll
            for (int cb = 0; cb < KT; ++cb) {
                const bf16x4 a = *reinterpret_cast<const bf16x4*>(mp + (16 * ct + r16) * DK + 16 * cb + 4 * g);
                s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, xb[cb], s, 0, 0, 0);
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const bf16x4 a = *reinterpret_cast<const bf16x4*>(qtT + (16 * ct + r16) * C + 16 * tb + 4 * g);
                s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, ob[tb], s, 0, 0, 0);
            }
            acc[ct] = s;
        }
    }
    if (p.ds0 != nullptr) {
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) stf4(p.ds0 + (static_cast<int64_t>(bh) * DV + v0 + r16) * DK + 16 * ct + 4 * g, acc[ct]);
    }
}

// ====================================================================== grads
// Per chunk (all natural-log gate gradients dG_i, summed back to d log alpha at the end):
//   dQt = dO S_in,  dM = S_in^T dS_out
//   dU0 = P^T dO + diag(w) K dS_out^T,   dP = dO U0^T - dQt W^T
//   dW  = -P^T dQt - diag(w) K dM^T
//   dK <- diag(w) (U0 dS_out - W dM),    dw_j = (U0 dS_out - W dM)_j . k_j
//   T^T dW, T^T dU0;  dT = dW (diag(beta g) K)^T + dU0 (diag(beta) V)^T
//   dA = strictly_lower(-T^T dT T^T),  KG = (K K^T . Gamma) strictly lower
//   dK <- M1 K + M1^T K with M1 = dA . diag(beta) KG-shape factors beta_i Gamma_ij
//   dP masked and decayed: dQ <- (dP . Gamma) K, dK <- (dP . Gamma)^T Q
//   dQ <- diag(g) dQt;  dK <- diag(beta g) T^T dW;  dV = diag(beta) T^T dU0
//   dbeta_i = g_i (T^T dW)_i . k_i + (T^T dU0)_i . v_i + sum_j dA_ij KG_ij
//   dG_i += g_i (dQt_i . q_i + beta_i (T^T dW)_i . k_i) + sum_j (dA . A + dP . P)_ij
//           - sum_j (dA . A + dP . P)_ji - w_i dw_i;  dG_last += sum_j w_j dw_j + e^(G_last) tr(dM)
template <int C, int DK, int DV>
__global__ __launch_bounds__(256)
void grads_kernel(GdBwdParams p) {
    using S = GdScratch<C, DK, DV>;
    float* const sc = p.scratch + static_cast<int64_t>(blockIdx.x) * S::floats;
    __shared__ float sg[C], sw[C], sGl[C], sbe[C], sdG[C], sdw[C], sdb[C];
    __shared__ float sTr;
    __shared__ float sx[kSxFloats], sy[kSyFloats];
    const int tid = threadIdx.x;
    for (int chunk = blockIdx.x; chunk < p.chunks; chunk += gridDim.x) {
        const int bh = chunk / p.NC, c = chunk % p.NC;
        const int t0 = c * C, n = (p.T - t0 < C) ? (p.T - t0) : C;
        const int64_t tok0 = static_cast<int64_t>(bh) * p.T + t0;
        const u16* K = p.k + tok0 * DK;
        const u16* Q = p.q + tok0 * DK;
        const u16* V = p.v + tok0 * DV;
        const u16* dO = p.dout + tok0 * DV;
        const float* G = p.g + static_cast<int64_t>(chunk) * C;
        const u16* TU = p.tu + static_cast<int64_t>(chunk) * C * C;
        const u16* TF = p.tfull + static_cast<int64_t>(chunk) * C * C;
        const u16* Sin = p.sin + static_cast<int64_t>(chunk) * DV * DK;
        const u16* dSo = p.dso + static_cast<int64_t>(chunk) * DV * DK;
        if (tid < C) {
            sGl[tid] = G[tid];
            sg[tid] = ex2(G[tid]);
            sw[tid] = ex2(G[C - 1] - G[tid]);
            sbe[tid] = tid < n ? p.beta[tok0 + tid] : 0.f;
            sdG[tid] = 0.f;
            sdw[tid] = 0.f;
            sdb[tid] = 0.f;
        }
        if (tid == 0) sTr = 0.f;
        __syncthreads();
        auto kx = [&](int j, int a) { return j < n ? bf(K[j * DK + a]) : 0.f; };
        auto qx = [&](int i, int a) { return i < n ? bf(Q[i * DK + a]) : 0.f; };
        auto vx = [&](int j, int m) { return j < n ? bf(V[j * DV + m]) : 0.f; };
        auto ox = [&](int i, int m) { return i < n ? bf(dO[i * DV + m]) : 0.f; };
        auto gam = [&](int i, int j) { return ex2(sGl[i] - sGl[j]); };
        // ---- W, U0, P (as in the maps); dQt = dO S_in; dM = S_in^T dS_out
        gemm_lds<C, DK, C>(sx, sy, [&](int i, int j) { return bf(TU[i * C + j]); }, [&](int j, int a) { return sg[j] * kx(j, a); },
                  [&](int i, int a, float v) { sc[S::W + i * DK + a] = v; });
        gemm_lds<C, DV, C>(sx, sy, [&](int i, int j) { return bf(TU[i * C + j]); }, vx,
                  [&](int i, int m, float v) { sc[S::U0 + i * DV + m] = v; });
        gemm_lds<C, C, DK>(sx, sy, qx, [&](int a, int j) { return kx(j, a); },
                  [&](int i, int j, float v) { sc[S::P + i * C + j] = j <= i ? v * gam(i, j) : 0.f; });
        gemm_lds<C, DK, DV>(sx, sy, ox, [&](int m, int a) { return bf(Sin[m * DK + a]); },
                  [&](int i, int a, float v) { sc[S::DQT + i * DK + a] = v; });
        gemm_lds<DK, DK, DV>(sx, sy, [&](int a, int m) { return bf(Sin[m * DK + a]); }, [&](int m, int b) { return bf(dSo[m * DK + b]); },
                  [&](int a, int b, float v) {
                      sc[S::DM + a * DK + b] = v;
                      if (a == b) atomicAdd(&sTr, v);
                  });
        // KG = (K K^T . Gamma) strictly lower
        gemm_lds<C, C, DK>(sx, sy, kx, [&](int a, int j) { return kx(j, a); },
                  [&](int i, int j, float v) { sc[S::KG + i * C + j] = j < i ? v * gam(i, j) : 0.f; });
        __syncthreads();
        // ---- dU0 = P^T dO + diag(w) K dS_out^T (reduction over C tokens, then DK keys)
        gemm_lds<C, DV, C + DK>(sx, sy,
                  [&](int j, int x) { return x < C ? scr(sc + S::P + x * C + j) : sw[j] * kx(j, x - C); },
                  [&](int x, int m) { return x < C ? ox(x, m) : bf(dSo[m * DK + x - C]); },
                  [&](int j, int m, float v) { sc[S::DU0 + j * DV + m] = v; });
        // dP = dO U0^T - dQt W^T (reduction over DV values, then DK keys), masked and decayed
        gemm_lds<C, C, DV + DK>(sx, sy,
                  [&](int i, int x) { return x < DV ? ox(i, x) : -scr(sc + S::DQT + i * DK + x - DV); },
                  [&](int x, int j) { return x < DV ? scr(sc + S::U0 + j * DV + x) : scr(sc + S::W + j * DK + x - DV); },
                  [&](int i, int j, float v) { sc[S::DP + i * C + j] = j <= i ? v : 0.f; });
        // dW = -P^T dQt - diag(w) K dM^T
        gemm_lds<C, DK, C + DK>(sx, sy,
                  [&](int j, int x) { return x < C ? -scr(sc + S::P + x * C + j) : -sw[j] * kx(j, x - C); },
                  [&](int x, int a) { return x < C ? scr(sc + S::DQT + x * DK + a) : scr(sc + S::DM + a * DK + x - C); },
                  [&](int j, int a, float v) { sc[S::DW + j * DK + a] = v; });
        // U0 dS_out - W dM: dK's first part (times w) and dw
        gemm_lds<C, DK, DV + DK>(sx, sy,
                  [&](int j, int x) { return x < DV ? scr(sc + S::U0 + j * DV + x) : -scr(sc + S::W + j * DK + x - DV); },
                  [&](int x, int b) { return x < DV ? bf(dSo[x * DK + b]) : scr(sc + S::DM + (x - DV) * DK + b); },
                  [&](int j, int b, float v) {
                      sc[S::DKX + j * DK + b] = sw[j] * v;
                      atomicAdd(&sdw[j], v * kx(j, b));
                  });
        __syncthreads();
        // ---- T^T dW, T^T dU0; dT = dW (diag(beta g) K)^T + dU0 (diag(beta) V)^T
        gemm_lds<C, DK, C>(sx, sy, [&](int j, int i) { return bf(TF[i * C + j]); }, [&](int i, int a) { return scr(sc + S::DW + i * DK + a); },
                  [&](int j, int a, float v) { sc[S::TDW + j * DK + a] = v; });
        gemm_lds<C, DV, C>(sx, sy, [&](int j, int i) { return bf(TF[i * C + j]); }, [&](int i, int m) { return scr(sc + S::DU0 + i * DV + m); },
                  [&](int j, int m, float v) { sc[S::TDU + j * DV + m] = v; });
        gemm_lds<C, C, DK + DV>(sx, sy,
                  [&](int i, int x) { return x < DK ? scr(sc + S::DW + i * DK + x) : scr(sc + S::DU0 + i * DV + x - DK); },
                  [&](int x, int j) { return x < DK ? sbe[j] * sg[j] * kx(j, x) : sbe[j] * vx(j, x - DK); },
                  [&](int i, int j, float v) { sc[S::DT + i * C + j] = v; });
        __syncthreads();
        // ---- Z = T^T dT, then dA = strictly_lower(-Z T^T)
        gemm_lds<C, C, C>(sx, sy, [&](int i, int l) { return bf(TF[l * C + i]); }, [&](int l, int j) { return scr(sc + S::DT + l * C + j); },
                  [&](int i, int j, float v) { sc[S::Z + i * C + j] = v; });
        __syncthreads();
        gemm_lds<C, C, C>(sx, sy, [&](int i, int l) { return scr(sc + S::Z + i * C + l); }, [&](int l, int j) { return bf(TF[j * C + l]); },
                  [&](int i, int j, float v) { sc[S::DA + i * C + j] = j < i ? -v : 0.f; });
        __syncthreads();
        // ---- row and column terms of dbeta and dG from dA (A = diag(beta) KG) and dP (P),
        // one thread per token
        if (tid < C) {
            const int i = tid;
            float db = 0.f, dg = 0.f;
            for (int j = 0; j < C; ++j) {
                const float da = scr(sc + S::DA + i * C + j), kg = scr(sc + S::KG + i * C + j);
                db += da * kg;
                dg += da * kg * sbe[i] + scr(sc + S::DP + i * C + j) * scr(sc + S::P + i * C + j);
                const float dac = scr(sc + S::DA + j * C + i), kgc = scr(sc + S::KG + j * C + i);
                dg -= dac * kgc * sbe[j] + scr(sc + S::DP + j * C + i) * scr(sc + S::P + j * C + i);
            }
            sdb[i] += db;
            sdG[i] += dg;
        }
        // dQ2 = (dP . Gamma) K + 0 (the decayed dP's reduction over tokens j)
        gemm_lds<C, DK, C>(sx, sy, [&](int i, int j) { return scr(sc + S::DP + i * C + j) * (j <= i ? gam(i, j) : 0.f); },
                  [&](int j, int a) { return kx(j, a); }, [&](int i, int a, float v) { sc[S::DQ2 + i * DK + a] = v; });
        __syncthreads();
        // ---- dK: the first part + diag(beta g) T^T dW + M1 K + M1^T K + (dP . Gamma)^T Q, with
        // M1_ij = dA_ij beta_i Gamma_ij (reduction over 2C tokens, then C tokens of the decayed dP)
        gemm_lds<C, DK, 3 * C>(sx, sy,
                  [&](int j, int x) {
                      if (x < C) return scr(sc + S::DA + x * C + j) * sbe[x] * (j < x ? gam(x, j) : 0.f);   // M1^T
                      if (x < 2 * C) { const int l = x - C; return scr(sc + S::DA + j * C + l) * sbe[j] * (l < j ? gam(j, l) : 0.f); }
                      const int i = x - 2 * C;
                      return scr(sc + S::DP + i * C + j) * (j <= i ? gam(i, j) : 0.f);
                  },
                  [&](int x, int b) { return x < 2 * C ? kx(x < C ? x : x - C, b) : qx(x - 2 * C, b); },
                  [&](int j, int b, float v) {
                      const float dkv = v + scr(sc + S::DKX + j * DK + b) + sbe[j] * sg[j] * scr(sc + S::TDW + j * DK + b);
                      if (j < n) p.dk[(tok0 + j) * DK + b] = to_bf(dkv);
                  });
        // dQ = diag(g) dQt + dQ2, and the per-token reductions of dbeta and dG
        for (int idx = tid; idx < C * DK; idx += 256) {
            const int i = idx / DK, a = idx % DK;
            if (i < n) p.dq[(tok0 + i) * DK + a] = to_bf(sg[i] * scr(sc + S::DQT + idx) + scr(sc + S::DQ2 + idx));
        }
        for (int idx = tid; idx < C * DV; idx += 256) {
            const int j = idx / DV, m = idx % DV;
            if (j < n) p.dv[(tok0 + j) * DV + m] = to_bf(sbe[j] * scr(sc + S::TDU + idx));
        }
        __syncthreads();
        if (tid < C) {
            const int i = tid;
            float tk = 0.f, qq = 0.f, uv = 0.f;
            for (int a = 0; a < DK; ++a) {
                tk += scr(sc + S::TDW + i * DK + a) * kx(i, a);
                qq += scr(sc + S::DQT + i * DK + a) * qx(i, a);
            }
            for (int m = 0; m < DV; ++m) uv += scr(sc + S::TDU + i * DV + m) * vx(i, m);
            sdb[i] += sg[i] * tk + uv;
            sdG[i] += sg[i] * (qq + sbe[i] * tk) - sw[i] * sdw[i];
        }
        __syncthreads();
        // dG_last gets the carry weights' share and the fade of the entering memory; then d log
        // alpha_t = sum_{i >= t} dG_i (one wave, reverse inclusive scan by shuffles)
        if (tid < 64) {
            const int lane = tid;
            float x = lane < C ? sdG[lane] : 0.f;
            float wsum = lane < C ? sw[lane] * sdw[lane] : 0.f;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) wsum += __shfl_xor(wsum, off, 64);
            if (lane == C - 1) x += wsum + ex2(sGl[C - 1]) * sTr;
            // reverse inclusive scan over lanes 0 .. 63
            float y = x;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float t = __shfl_down(y, off, 64);
                if (lane + off < 64) y += t;
            }
            if (lane < n) {
                p.dalpha[tok0 + lane] = y;
                p.dbeta[tok0 + lane] = sdb[lane];
            }
        }
        __syncthreads();
    }
}

// ====================================================================== launch
template <int C, int DK, int DV>
hipError_t launch_gdelta_bwd_dv(const BwdArgs& a, hipStream_t stream) {
    const int NC = (a.T + C - 1) / C;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    const int64_t chunks = heads * NC;
    unsigned char* ws = static_cast<unsigned char*>(a.ws);
    auto take = [&](int64_t bytes) { unsigned char* q = ws; ws += delta_ws_align(bytes); return q; };
    GdBwdParams p{};
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.alpha = a.gate;
    p.beta = a.beta;
    p.s0 = a.s0;
    p.dout = static_cast<const u16*>(a.dout);
    p.ds_out = a.ds_out;
    p.dq = static_cast<u16*>(a.grad_q);
    p.dk = static_cast<u16*>(a.grad_k);
    p.dv = static_cast<u16*>(a.grad_v);
    p.dalpha = a.dgate;
    p.dbeta = a.dbeta;
    p.ds0 = a.ds0;
    u16* tu = reinterpret_cast<u16*>(take(chunks * C * C * 2));
    float* g = reinterpret_cast<float*>(take(chunks * C * 4));
    u16* tfull = reinterpret_cast<u16*>(take(chunks * C * C * 2));
    p.tu = tu;
    p.g = g;
    p.tfull = tfull;
    p.qtT = reinterpret_cast<u16*>(take(chunks * DK * C * 2));
    p.mp = reinterpret_cast<u16*>(take(chunks * DK * DK * 2));
    p.mpT = reinterpret_cast<u16*>(take(chunks * DK * DK * 2));
    p.nn = reinterpret_cast<u16*>(take(chunks * DV * DK * 2));
    p.sin = reinterpret_cast<u16*>(take(chunks * DV * DK * 2));
    p.dso = reinterpret_cast<u16*>(take(chunks * DV * DK * 2));
    p.T = a.T;
    p.NC = NC;
    p.chunks = static_cast<int>(chunks);
    if (chunks == 0) {
        // T == 0: ds0 = ds_out (or zeros), no token gradients
        if (a.ds0 != nullptr) {
            const size_t bytes = static_cast<size_t>(heads) * DV * DK * 4;
            if (a.ds_out != nullptr) return hipMemcpyAsync(a.ds0, a.ds_out, bytes, hipMemcpyDeviceToDevice, stream);
            return hipMemsetAsync(a.ds0, 0, bytes, stream);
        }
        return hipSuccess;
    }
    // the prep's parameters: T_U, G and T of every chunk
    DspParams tp{};
    tp.q = p.q;
    tp.k = p.k;
    tp.alpha = a.gate;
    tp.beta = a.beta;
    tp.tu = tu;
    tp.g = g;
    tp.tfull = tfull;
    tp.qraw = p.q;
    tp.kraw = p.k;
    tp.T = a.T;
    tp.NC = NC;
    tp.map = 0;
    hipLaunchKernelGGL((delta_tfac_kernel<C, DK>), dim3(static_cast<unsigned>(chunks)), dim3(256), 0, stream, tp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned wgs = static_cast<unsigned>(gd_bwd_workgroups(chunks));
    u16* rec_u = reinterpret_cast<u16*>(take(chunks * C * DV * 2));
    u16* rec_r = reinterpret_cast<u16*>(take(chunks * C * DV * 2));
    u16* rec_du = reinterpret_cast<u16*>(take(chunks * C * DV * 2));
    p.scratch = reinterpret_cast<float*>(ws);
    bool single = false;
    if constexpr (C == 64 && DK >= 32) single = delta_sp_fits(a.T, DK, DV);
    if (single) {
        if constexpr (C == 64 && DK >= 32) {
            // the forward single pass recording S_in, U and R per chunk; then the same pass in
            // reverse for dS' and dU per chunk, dV and ds0
            constexpr int VS = DV >= 32 ? 32 : 16;
            DspParams fp{};
            fp.q = p.q;
            fp.k = p.k;
            fp.v = p.v;
            fp.alpha = a.gate;
            fp.beta = a.beta;
            fp.s0 = a.s0;
            fp.tu = tu;
            fp.g = g;
            fp.T = a.T;
            fp.NC = NC;
            fp.qk_seq = a.T;
            fp.slices = DV / VS;
            const int64_t grid = heads * fp.slices;
            fp.remap = (grid % 8 == 0) ? 1 : 0;
            DspParams rp = fp;
            fp.st_s = p.sin;
            fp.st_u = rec_u;
            fp.st_r = rec_r;
            hipLaunchKernelGGL((delta_sp_kernel<C, DK, DV, VS, kGateDeltaRule, 1, false, true>), dim3(static_cast<unsigned>(grid)),
                               dim3(256), 0, stream, fp);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            rp.v = p.dout;
            rp.s0 = a.ds_out;
            rp.o = p.dv;
            rp.s_out = a.ds0;
            rp.st_s = p.dso;
            rp.st_u = rec_du;
            hipLaunchKernelGGL((delta_sp_kernel<C, DK, DV, VS, kGateDeltaRule, 1, true>), dim3(static_cast<unsigned>(grid)),
                               dim3(256), 0, stream, rp);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            if constexpr (DV % 32 == 0) {
                p.rec_u = rec_u;
                p.rec_r = rec_r;
                p.rec_du = rec_du;
                hipLaunchKernelGGL((gd_grads_kernel<DK, DV>), dim3(static_cast<unsigned>(gd_grads_workgroups(chunks))), dim3(512), 0,
                                   stream, p);
                return hipGetLastError();
            }
        }
    } else {
        hipLaunchKernelGGL((maps_kernel<C, DK, DV>), dim3(wgs), dim3(256), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const unsigned rows = static_cast<unsigned>(heads * (DV / 16));
        hipLaunchKernelGGL((fwd_chain_kernel<C, DK, DV>), dim3(rows), dim3(64), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL((bwd_chain_kernel<C, DK, DV>), dim3(rows), dim3(64), 0, stream, p);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    hipLaunchKernelGGL((grads_kernel<C, DK, DV>), dim3(wgs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int C, int DK>
hipError_t launch_gdelta_bwd_dk(const BwdArgs& a, hipStream_t stream) {
    switch (a.dv) {
        case 16: return launch_gdelta_bwd_dv<C, DK, 16>(a, stream);
        case 32: return launch_gdelta_bwd_dv<C, DK, 32>(a, stream);
        case 64: return launch_gdelta_bwd_dv<C, DK, 64>(a, stream);
        case 128: return launch_gdelta_bwd_dv<C, DK, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

template <int C>
hipError_t launch_gdelta_bwd(const BwdArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_gdelta_bwd_dk<C, 16>(a, stream);
        case 32: return launch_gdelta_bwd_dk<C, 32>(a, stream);
        case 64: return launch_gdelta_bwd_dk<C, 64>(a, stream);
        case 128: return launch_gdelta_bwd_dk<C, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
