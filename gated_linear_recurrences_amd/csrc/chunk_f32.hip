// Chunkwise forward in float32 storage and fp32 arithmetic (VALU), all four
// gate variants.
//
// The chunkwise form of "Le architetture lineari: RetNet, RWKV, xLSTM"
// (section "RetNet: la retention e le sue tre forme", Fig. 16.5): inside a
// chunk of n tokens the masked-decay triangle is evaluated in parallel, and the
// memory at the end of the chunk is handed to the next one. With local index
// i, j in [0, n), incoming memory S_in and local inclusive cumulative
// log-gates (b for the per-channel gate, G for the scalar one):
//
//   retention  o_i = sum_{j<=i} g^(i-j) (q_i.k_j) v_j + g^(i+1) S_in q_i
//              S_out = g^n S_in + sum_j g^(n-1-j) v_j k_j^T
//   scalar     (data-dependent, one gate per token) the same with g^(i-j) -> e^(G_i - G_j):
//              o_i = sum_{j<=i} e^(G_i - G_j) (q_i.k_j) v_j + e^(G_i) S_in q_i
//              S_out = e^(G_{n-1}) S_in + sum_j e^(G_{n-1} - G_j) v_j k_j^T
//   GLA        o_i = sum_{j<=i} [sum_c q_ic k_jc e^(b_ic - b_jc)] v_j + S_in (q_i . e^(b_i))
//              S_out = S_in Diag(e^(b_{n-1})) + sum_j v_j (k_j . e^(b_{n-1} - b_j))^T
//   gated delta (WY form; "Scrivere meglio nella memoria", sections "Correggere:
//              la delta rule" and "Unire oblio e correzione"):
//              (I + A) U = diag(beta) (V - diag(e^G) K S_in^T),
//              A = strictly_lower(diag(beta) (K K^T . Gamma)), Gamma_ij = e^(G_i - G_j)
//              o_i = e^(G_i) S_in q_i + sum_{j<=i} Gamma_ij (q_i.k_j) u_j
//              S_out = e^(G_{n-1}) S_in + sum_j e^(G_{n-1} - G_j) u_j k_j^T
//
// This path exists for float32 callers and small heads; it favours plain,
// exact fp32 arithmetic (one exponential per decayed term) over speed. One
// workgroup owns one (batch, head) and a tile of DVT value channels: the rows
// of S evolve independently in every variant (gates act on key channels), so
// value-channel tiles never communicate.
#include "device_common.hpp"
#include "launch.hpp"

namespace glr {

namespace {

constexpr int kThreads = 256;

template <int VARIANT, int C, int DK, int DVT>
__global__ __launch_bounds__(kThreads)
void chunk_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                      const float* __restrict__ v, const float* __restrict__ gate,
                      const float* __restrict__ beta, const float* __restrict__ s0,
                      float* __restrict__ o, float* __restrict__ s_out,
                      int H, int T, int dv, int fuse) {
    __shared__ float Qs[C][DK + 1];
    __shared__ float Ks[C][DK + 1];
    __shared__ float Vs[C][DVT + 1];          // values; pseudo-values u for the delta rule
    __shared__ float Ss[DVT][DK + 1];         // memory tile, rows = value channels
    __shared__ float Ps[C][C + 1];            // decayed causal scores
    __shared__ float Bs[VARIANT == kGLA ? C : 1][DK + 1];      // GLA cumulative log-gates
    __shared__ float As[VARIANT == kGDelta ? C : 1][C + 1];    // delta-rule triangular system
    __shared__ float Gs[C], Betas[C];

    const int tiles = dv / DVT;
    const int bh = blockIdx.x / tiles;
    const int v0 = (blockIdx.x % tiles) * DVT;
    const int h = bh % H;
    const int tid = threadIdx.x;
    const int64_t base_k = static_cast<int64_t>(bh) * T * DK;
    const int64_t base_v = static_cast<int64_t>(bh) * T * dv;
    const int64_t base_s = static_cast<int64_t>(bh) * dv * DK;
    const float lg = (VARIANT == kRetention) ? gate[h] : 0.f;

    for (int e = tid; e < DVT * DK; e += kThreads) {
        const int m = e / DK, c = e % DK;
        Ss[m][c] = s0 ? s0[base_s + static_cast<int64_t>(v0 + m) * DK + c] : 0.f;
    }

    for (int t0 = 0; t0 < T; t0 += C) {
        const int n = min(C, T - t0);
        __syncthreads();  // previous chunk fully consumed
        for (int e = tid; e < C * DK; e += kThreads) {
            const int i = e / DK, c = e % DK;
            const bool in = i < n;
            const int64_t off = base_k + static_cast<int64_t>(t0 + i) * DK + c;
            Qs[i][c] = in ? q[off] : 0.f;
            Ks[i][c] = in ? k[off] : 0.f;
        }
        for (int e = tid; e < C * DVT; e += kThreads) {
            const int i = e / DVT, m = e % DVT;
            Vs[i][m] = (i < n) ? v[base_v + static_cast<int64_t>(t0 + i) * dv + v0 + m] : 0.f;
        }
        if constexpr (VARIANT == kGLA) {
            // inclusive cumulative sum of the log-gates along the chunk, one key channel per thread
            for (int c = tid; c < DK; c += kThreads) {
                float acc = 0.f;
                for (int i = 0; i < C; ++i) {
                    if (i < n) acc += gate[base_k + static_cast<int64_t>(t0 + i) * DK + c];
                    Bs[i][c] = acc;
                }
            }
        }
        if constexpr (VARIANT == kGDelta) {
            if (fuse & 1) {
                // DeltaNet's feature map on q and k: SiLU, then unit L2 norm per token
                __syncthreads();
                for (int r = tid; r < 2 * C; r += kThreads) {
                    float* row = (r < C) ? Qs[r] : Ks[r - C];
                    float ss = 0.f;
                    for (int c = 0; c < DK; ++c) {
                        const float y = row[c] / (1.f + __expf(-row[c]));
                        row[c] = y;
                        ss += y * y;
                    }
                    const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
                    for (int c = 0; c < DK; ++c) row[c] *= inv;
                }
            }
        }
        if constexpr (VARIANT == kGDelta || VARIANT == kScalar) {
            if (tid == 0) {
                float acc = 0.f;
                const int64_t base_t = static_cast<int64_t>(bh) * T + t0;
                for (int i = 0; i < C; ++i) {
                    if (i < n) acc += gate[base_t + i];
                    Gs[i] = acc;
                    Betas[i] = (VARIANT == kGDelta && i < n) ? beta[base_t + i] : 0.f;
                }
            }
        }
        __syncthreads();

        // decayed causal scores (and the delta rule's triangular system)
        for (int e = tid; e < C * C; e += kThreads) {
            const int i = e / C, j = e % C;
            float p = 0.f, a = 0.f;
            if (j <= i && i < n) {
                if constexpr (VARIANT == kGLA) {
                    for (int c = 0; c < DK; ++c) p += Qs[i][c] * Ks[j][c] * __expf(Bs[i][c] - Bs[j][c]);
                } else {
                    float qk = 0.f, kk = 0.f;
                    for (int c = 0; c < DK; ++c) {
                        qk += Qs[i][c] * Ks[j][c];
                        if (VARIANT == kGDelta) kk += Ks[i][c] * Ks[j][c];
                    }
                    const float dec = (VARIANT == kRetention) ? __expf(lg * static_cast<float>(i - j))
                                                              : __expf(Gs[i] - Gs[j]);
                    p = qk * dec;
                    a = (j < i) ? Betas[i] * kk * dec : 0.f;
                }
            }
            Ps[i][j] = p;
            if constexpr (VARIANT == kGDelta) As[i][j] = a;
        }
        __syncthreads();

        if constexpr (VARIANT == kGDelta) {
            // right-hand side beta_i (v_i - e^{G_i} S_in k_i), then forward substitution
            for (int e = tid; e < C * DVT; e += kThreads) {
                const int i = e / DVT, m = e % DVT;
                float sk = 0.f;
                for (int c = 0; c < DK; ++c) sk += Ss[m][c] * Ks[i][c];
                Vs[i][m] = Betas[i] * (Vs[i][m] - __expf(Gs[i]) * sk);
            }
            __syncthreads();
            for (int m = tid; m < DVT; m += kThreads) {
                for (int i = 1; i < n; ++i) {
                    float acc = Vs[i][m];
                    for (int j = 0; j < i; ++j) acc -= As[i][j] * Vs[j][m];
                    Vs[i][m] = acc;
                }
            }
            __syncthreads();
        }

        // outputs: intra-chunk triangle plus the readout of the incoming memory
        for (int e = tid; e < n * DVT; e += kThreads) {
            const int i = e / DVT, m = e % DVT;
            float acc = 0.f;
            for (int j = 0; j <= i; ++j) acc += Ps[i][j] * Vs[j][m];
            float rd = 0.f;
            if constexpr (VARIANT == kGLA) {
                for (int c = 0; c < DK; ++c) rd += Ss[m][c] * Qs[i][c] * __expf(Bs[i][c]);
            } else {
                for (int c = 0; c < DK; ++c) rd += Ss[m][c] * Qs[i][c];
                rd *= (VARIANT == kRetention) ? __expf(lg * static_cast<float>(i + 1)) : __expf(Gs[i]);
            }
            o[base_v + static_cast<int64_t>(t0 + i) * dv + v0 + m] = acc + rd;
        }
        __syncthreads();

        // memory handed to the next chunk
        for (int e = tid; e < DVT * DK; e += kThreads) {
            const int m = e / DK, c = e % DK;
            float acc;
            if constexpr (VARIANT == kGLA) {
                const float last = Bs[n - 1][c];
                acc = Ss[m][c] * __expf(last);
                for (int j = 0; j < n; ++j) acc += Vs[j][m] * Ks[j][c] * __expf(last - Bs[j][c]);
            } else {
                const float last = (VARIANT == kRetention) ? lg * static_cast<float>(n - 1) : Gs[n - 1];
                acc = Ss[m][c] * __expf((VARIANT == kRetention) ? lg * static_cast<float>(n) : last);
                for (int j = 0; j < n; ++j) {
                    const float w = (VARIANT == kRetention) ? __expf(lg * static_cast<float>(n - 1 - j))
                                                            : __expf(last - Gs[j]);
                    acc += w * Vs[j][m] * Ks[j][c];
                }
            }
            Ss[m][c] = acc;
        }
    }
    __syncthreads();
    if (s_out) {
        for (int e = tid; e < DVT * DK; e += kThreads) {
            const int m = e / DK, c = e % DK;
            s_out[base_s + static_cast<int64_t>(v0 + m) * DK + c] = Ss[m][c];
        }
    }
}

// RMS norm of each output row (the gated delta rule's fused epilogue in fp32): one
// wave per row, the sum of squares by shuffles.
__global__ __launch_bounds__(256)
void rms_rows_f32(float* __restrict__ o, const float* __restrict__ w, float eps, int64_t rows, int dv) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    float* r = o + row * dv;
    float ss = 0.f;
    for (int c = lane; c < dv; c += 64) ss += r[c] * r[c];
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.f / sqrtf(ss / static_cast<float>(dv) + eps);
    for (int c = lane; c < dv; c += 64) r[c] = r[c] * w[c] * inv;
}

// Layer norm of each output row (GLA's fused epilogue in fp32): one wave per row, the mean
// and then the squared deviations by shuffles.
__global__ __launch_bounds__(256)
void layernorm_rows_f32(float* __restrict__ o, const float* __restrict__ w, const float* __restrict__ b, float eps,
                        int64_t rows, int dv) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    float* r = o + row * dv;
    float s = 0.f;
    for (int c = lane; c < dv; c += 64) s += r[c];
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const float mean = s / static_cast<float>(dv);
    float ss = 0.f;
    for (int c = lane; c < dv; c += 64) ss += (r[c] - mean) * (r[c] - mean);
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.f / sqrtf(ss / static_cast<float>(dv) + eps);
    for (int c = lane; c < dv; c += 64) r[c] = (r[c] - mean) * inv * w[c] + (b ? b[c] : 0.f);
}

template <int VARIANT, int C, int DK>
hipError_t launch_dk(const ChunkArgs& a, hipStream_t stream) {
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* o = static_cast<float*>(a.o);
    const int bh = a.B * a.H;
    if (a.dv >= 32) {
        const dim3 grid(bh * (a.dv / 32));
        hipLaunchKernelGGL((chunk_f32_kernel<VARIANT, C, DK, 32>), grid, dim3(kThreads), 0, stream,
                           q, k, v, a.gate, a.beta, a.s0, o, a.s_out, a.H, a.T, a.dv, a.fuse);
    } else {
        const dim3 grid(bh);
        hipLaunchKernelGGL((chunk_f32_kernel<VARIANT, C, DK, 16>), grid, dim3(kThreads), 0, stream,
                           q, k, v, a.gate, a.beta, a.s0, o, a.s_out, a.H, a.T, a.dv, a.fuse);
    }
    hipError_t err = hipGetLastError();
    const int64_t rows = static_cast<int64_t>(bh) * a.T;
    if (err != hipSuccess || !(a.fuse & 6) || rows == 0) return err;
    if (a.fuse & 4)
        hipLaunchKernelGGL(layernorm_rows_f32, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, o,
                           a.onw, a.onb, a.oeps, rows, a.dv);
    else
        hipLaunchKernelGGL(rms_rows_f32, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, o, a.onw,
                           a.oeps, rows, a.dv);
    return hipGetLastError();
}

template <int VARIANT, int C>
hipError_t launch_c(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_dk<VARIANT, C, 16>(a, stream);
        case 32: return launch_dk<VARIANT, C, 32>(a, stream);
        case 64: return launch_dk<VARIANT, C, 64>(a, stream);
        case 128: return launch_dk<VARIANT, C, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int VARIANT>
hipError_t launch_variant(const ChunkArgs& a, hipStream_t stream) {
    switch (a.chunk) {
        case 16: return launch_c<VARIANT, 16>(a, stream);
        case 32: return launch_c<VARIANT, 32>(a, stream);
        case 64: return launch_c<VARIANT, 64>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_f32(Variant variant, const ChunkArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    switch (variant) {
        case kRetention: return launch_variant<kRetention>(a, stream);
        case kGLA: return launch_variant<kGLA>(a, stream);
        case kGDelta: return launch_variant<kGDelta>(a, stream);
        case kScalar: return launch_variant<kScalar>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace glr
