// Single-token decode: S <- S Diag(alpha); S <- S + v k^T; o = S q, and the same
// step under the gated delta rule: S <- S [alpha (I - beta k k^T)] + beta v k^T.
//
// The recurrent form of retention ("Le architetture lineari: RetNet, RWKV,
// xLSTM", section "RetNet: la retention e le sue tre forme"): every token costs
// the same two gestures on a memory of constant size. With a gate per key
// channel this is the GLA row of the transition table ("Scrivere meglio nella
// memoria", section "Le ricorrenze come regressione online").
//
// The step is a pure stream of the fp32 memory: 2 * d_v * d_k * 4 bytes per
// (sequence, head) against ~5 d_v d_k flops, far below the machine balance, so
// the design goal is HBM bandwidth: one workgroup per (sequence, head) sized so
// each thread owns about eight 16-byte pieces of S (512 threads at d = 128),
// all loaded before any is used; non-temporal loads/stores (measured 13% faster
// than cached ones on this stream); each row of S owned by a group of d_k/4
// lanes that reduce the readout with cross-lane shuffles.
//
// Gated delta rule ("Scrivere meglio nella memoria", section "Unire oblio e
// correzione: Gated DeltaNet"), one gate alpha and one write strength beta per
// (sequence, head). Per row m of S, from the old row: e = S_m . k (what the
// memory reads under k) and r = S_m . q, both reduced over the row's lane group;
// then u = beta (v_m - alpha e), the new row alpha S_m + u k^T, and the readout
// o_m = alpha r + u (k . q). The row is read and written once, as above.
#include "device_common.hpp"
#include "launch.hpp"

namespace glr {

namespace {

// threads per (sequence, head): eight 16-byte pieces of S per thread, 64..512
template <int DK, int DV>
constexpr int decode_threads() {
    return (DK * DV / 32 < 64) ? 64 : ((DK * DV / 32 > 512) ? 512 : DK * DV / 32);
}

template <typename TS, int DK, int DV, bool DELTA>
__global__ __launch_bounds__((decode_threads<DK, DV>()))
void decode_step_kernel(const TS* __restrict__ q, const TS* __restrict__ k, const TS* __restrict__ v,
                        const float* __restrict__ alpha, const float* __restrict__ beta, float* __restrict__ s,
                        TS* __restrict__ o) {
    constexpr int kThreads = decode_threads<DK, DV>();
    constexpr int kLanesPerRow = DK / 4;                      // each lane owns 4 key channels
    constexpr int kRowsPerPass = kThreads / kLanesPerRow;
    // every row a thread owns is loaded before any is used: all of them in flight at once
    constexpr int kRows = (DV + kRowsPerPass - 1) / kRowsPerPass;
    const int64_t pair = blockIdx.x;                          // (sequence, head)
    const int tid = threadIdx.x;
    const int c0 = (tid % kLanesPerRow) * 4;
    const int row = tid / kLanesPerRow;

    float* S = s + pair * static_cast<int64_t>(DV) * DK;
    f32x4 x[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int m = row + r * kRowsPerPass;
        if (m < DV) x[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + m * DK + c0));
    }
    const int64_t tok_k = pair * DK;
    const int64_t tok_v = pair * DV;
    float qc[4], kc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        qc[e] = Store<TS>::load(q, tok_k + c0 + e);
        kc[e] = Store<TS>::load(k, tok_k + c0 + e);
    }
    f32x4 ac = {1.f, 1.f, 1.f, 1.f};
    float a_s = 1.f, b_s = 0.f, kq = 0.f;
    if constexpr (DELTA) {
        a_s = alpha[pair];
        b_s = beta[pair];
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) t += kc[e] * qc[e];
        kq = group_sum<kLanesPerRow>(t);
    } else {
        ac = *reinterpret_cast<const f32x4*>(alpha + tok_k + c0);
    }
    float vm[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int m = row + r * kRowsPerPass;
        vm[r] = (m < DV) ? Store<TS>::load(v, tok_v + m) : 0.f;
    }

#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int m = row + r * kRowsPerPass;
        if (kRows * kRowsPerPass > DV && m >= DV) continue;   // only when DV < rows per pass
        float dot = 0.f;
        if constexpr (DELTA) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk += x[r][e] * kc[e];
                sq += x[r][e] * qc[e];
            }
            sk = group_sum<kLanesPerRow>(sk);
            sq = group_sum<kLanesPerRow>(sq);
            const float u = b_s * (vm[r] - a_s * sk);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[r][e] = a_s * x[r][e] + u * kc[e];
            dot = a_s * sq + u * kq;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[r][e] = x[r][e] * ac[e] + vm[r] * kc[e];
                dot += x[r][e] * qc[e];
            }
        }
        __builtin_nontemporal_store(x[r], reinterpret_cast<f32x4*>(S + m * DK + c0));
        if constexpr (!DELTA) dot = group_sum<kLanesPerRow>(dot);
        if ((tid % kLanesPerRow) == 0) Store<TS>::store(o, tok_v + m, dot);
    }
}

template <typename TS, int DK, bool DELTA>
hipError_t launch_dk(const DecodeArgs& a, const dim3& grid, hipStream_t stream) {
    const TS* q = static_cast<const TS*>(a.q);
    const TS* k = static_cast<const TS*>(a.k);
    const TS* v = static_cast<const TS*>(a.v);
    TS* o = static_cast<TS*>(a.o);
    switch (a.dv) {
        case 16: hipLaunchKernelGGL((decode_step_kernel<TS, DK, 16, DELTA>), grid, dim3(decode_threads<DK, 16>()), 0, stream, q, k, v, a.alpha, a.beta, a.s, o); break;
        case 32: hipLaunchKernelGGL((decode_step_kernel<TS, DK, 32, DELTA>), grid, dim3(decode_threads<DK, 32>()), 0, stream, q, k, v, a.alpha, a.beta, a.s, o); break;
        case 64: hipLaunchKernelGGL((decode_step_kernel<TS, DK, 64, DELTA>), grid, dim3(decode_threads<DK, 64>()), 0, stream, q, k, v, a.alpha, a.beta, a.s, o); break;
        case 128: hipLaunchKernelGGL((decode_step_kernel<TS, DK, 128, DELTA>), grid, dim3(decode_threads<DK, 128>()), 0, stream, q, k, v, a.alpha, a.beta, a.s, o); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename TS, bool DELTA>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
    const int64_t pairs = static_cast<int64_t>(a.N) * a.H;
    if (pairs == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(pairs));
    switch (a.dk) {
        case 16: return launch_dk<TS, 16, DELTA>(a, grid, stream);
        case 32: return launch_dk<TS, 32, DELTA>(a, grid, stream);
        case 64: return launch_dk<TS, 64, DELTA>(a, grid, stream);
        case 128: return launch_dk<TS, 128, DELTA>(a, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(bool bf16, const DecodeArgs& a, hipStream_t stream) {
    if (a.beta != nullptr)
        return bf16 ? launch_typed<unsigned short, true>(a, stream) : launch_typed<float, true>(a, stream);
    return bf16 ? launch_typed<unsigned short, false>(a, stream) : launch_typed<float, false>(a, stream);
}

}  // namespace glr
