// GLA's chunked forward in one pass (bf16 storage, chunk 64, d_k of 32, 64 or 128).
//
// Method: GLA's per-channel gated memory ("Scrivere meglio nella memoria", section
// "Dimenticare: i gate") in the chunkwise form of retention ("Le architetture lineari: RetNet,
// RWKV, xLSTM", section "RetNet: la retention e le sue tre forme", Fig. 16.5). The memory decays
// per key channel: S_t = S_{t-1} diag(alpha_t) + v_t k_t^T and o_t = S_t q_t. Over a chunk with
// chunk-local inclusive cumulative log2-gates B_t (one per key channel) and the memory S_in
// entering it:
//   o_t   = S_in (q_t . 2^B_t) + sum_{s <= t} [sum_c q_tc k_sc 2^(B_tc - B_sc)] v_s
//   S_out = S_in diag(2^B_last) + sum_s v_s (k_s . 2^(B_last - B_s))^T
//
// The workgroup is the gated delta rule's single pass (chunk_delta_sp.hpp) without its delta
// step: one workgroup of four waves per (sequence, value slice of VS channels). Chain waves 0
// and 1 hold S^T of their value tiles in fp32 MFMA accumulators across the chunks; helper
// waves 2 and 3 make the next chunk's operands while the chain works on the current one, one
// barrier per chunk. What differs is the helpers' share, which carries the per-channel gates:
//   - helper h owns key channels [h d_k / 2, (h + 1) d_k / 2). Lane (r, g) loads KPL = d_k / 32
//     of them for the 16 tokens of token tile g (q and k as 2 KPL-byte pieces, the raw log
//     gates as 4 KPL-byte pieces), so the scan of the gates runs along the lane's registers
//     and across the four tiles by two shuffles;
//   - per token tile and key, the reference m is the cumulative gate just before the tile,
//     lowered to 80 nats above the tile's last one when the tile decays more than that, so
//     that q 2^(B - m) and k 2^(m - B) stay finite for tiles down to -160 nats. The chain's
//     operands follow from them by one factor each: q 2^B = (q 2^(B - m)) 2^m and
//     k 2^(B_last - B) = (k 2^(m - B)) 2^(B_last - m), both at most |q| and |k|;
//   - each helper forms the causal triangle over its own key half, tile pairs (it, jt < it)
//     joined by F = 2^(m_it - m_jt) <= 1 on the q operand, so the helpers never wait for
//     each other; the chain adds the two partial triangles in its products with v.
// The chain's work per chunk is then that of the scalar decay with the decay of S^T taken
// per key (one factor per accumulator) and the token weights already inside the operands.
//
// LDS (d_k 128, 64-channel slices): the chain's two operands in two slots, the helpers' two
// in one (each helper reads back only what it wrote), 2^B_last in two slots, the F tables,
// the v slice in two slots and the partial triangles in two slots per helper: 152 KB.
// Buffer offsets are 31-bit: one sequence's raw gates (rows padded to whole chunks times d_k
// times 4 bytes), q, k, v and o must stay below 2^31 bytes.
#pragma once

#include "chunk_common.hpp"

namespace glr {
namespace ck {

struct GspParams {
    const u16* q;         // [BH][T][DK]
    const u16* k;         // [BH][T][DK]
    const u16* v;         // [BH][T][DV]
    const float* alpha;   // log alpha [BH][T][DK]
    const float* s0;      // [BH][DV][DK] or null
    u16* o;               // [BH][T][DV]
    float* s_out;         // [BH][DV][DK] or null
    int T, NC, slices, remap;
};

template <int DK, int VS>
struct GspLayout {
    static constexpr int C = 64;
    using TK = SwzTile<DK>;     // q and k rows (and their rescaled forms)
    using TV = SwzTile<VS>;     // the v slice
    static constexpr int RS = C + 8;
    static constexpr int HALF = DK / 2;
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int KBUF = al(C * TK::STRIDE * 2);
    static constexpr int VBUF = al(C * TV::STRIDE * 2);
    static constexpr int RBUF = al(C * RS * 2);
    static constexpr int EBUF = al(DK * 4);
    static constexpr int FBUF = al(6 * HALF * 4);
    static constexpr int oK = 0;                 // k 2^(B_last - B): the chain's, two slots
    static constexpr int oQ = oK + 2 * KBUF;     // q 2^B: the chain's, two slots
    static constexpr int oKh = oQ + 2 * KBUF;    // k 2^(m - B): the helpers', one slot
    static constexpr int oQh = oKh + KBUF;       // q 2^(B - m): the helpers', one slot
    static constexpr int oE = oQh + KBUF;        // 2^B_last per key, two slots
    static constexpr int oF = oE + 2 * EBUF;     // F per helper: [pair][key of its half]
    static constexpr int oV = oF + 2 * FBUF;     // the v slice, two slots
    static constexpr int oP = oV + 2 * VBUF;     // partial triangles [slot][helper]
    static constexpr int bytes = oP + 4 * RBUF;
    static_assert(bytes <= 160 * 1024, "LDS budget of the GLA single pass exceeded");
};

// One sequence's buffers within 31-bit offsets (rows padded to whole chunks).
inline bool gla_sp_fits(int T, int dk, int dv) {
    const long long rows = (static_cast<long long>(T) + 63) / 64 * 64;
    const long long per_row = dk * 4 > dv * 2 ? dk * 4 : dv * 2;
    return rows * per_row < (1ll << 31);
}

// bf16 element e (e < 2) of a packed pair, as float
__device__ __forceinline__ float bf_at(unsigned x, int e) {
    return __builtin_bit_cast(float, e ? (x & 0xffff0000u) : (x << 16));
}

template <int DK, int DV, int VS, int VW>
__global__ __launch_bounds__(256)
void gla_sp_kernel(GspParams p) {
    constexpr int C = 64;
    using Lay = GspLayout<DK, VS>;
    using TK = typename Lay::TK;
    using TV = typename Lay::TV;
    constexpr int NV = VS / 16;
    constexpr int CT = C / 16, JB = CT / 2;     // token tiles, 32-token blocks
    constexpr int KT = DK / 16, KB = DK / 32;   // key tiles, 32-key blocks
    constexpr int RS = Lay::RS;
    constexpr int HALF = Lay::HALF;             // keys per helper
    constexpr int KPL = HALF / 16;              // keys per helper lane
    constexpr int QD = KPL >= 2 ? KPL / 2 : 1;  // 32-bit words of a lane's q or k piece
    constexpr int KBH = HALF >= 32 ? HALF / 32 : 1;   // 32-key blocks of a helper's triangle
    constexpr int NH = 128;                     // helper threads
    constexpr int PV = C * VS / 8, NVP = (PV + NH - 1) / NH;
    static_assert(DK == 32 || DK == 64 || DK == 128, "d_k of 32, 64 or 128");
    static_assert(DV % VS == 0 && (VS == 16 * VW || VS == 32 * VW), "value slices of one or two chain waves");
    static_assert(PV <= 4 * NH, "v pieces per helper thread");

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    auto sK = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oK + (b & 1) * Lay::KBUF); };
    auto sQ = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oQ + (b & 1) * Lay::KBUF); };
    auto sE = [&](int b) { return reinterpret_cast<float*>(smem + Lay::oE + (b & 1) * Lay::EBUF); };
    auto sV = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oV + (b & 1) * Lay::VBUF); };
    auto sP = [&](int b, int h) { return reinterpret_cast<u16*>(smem + Lay::oP + (2 * (b & 1) + h) * Lay::RBUF); };
    u16* const sKh = reinterpret_cast<u16*>(smem + Lay::oKh);
    u16* const sQh = reinterpret_cast<u16*>(smem + Lay::oQh);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    // key channels held by a chain wave's memory tile ct at lane group g: chan(ct) + e, e < 4
    // (the bf16 operand built from tiles 2b and 2b + 1 holds keys 32b + 8g + 0..7)
    auto chan = [&](int ct) { return 32 * (ct >> 1) + 8 * g + 4 * (ct & 1); };
    const int lb = logical_block_of(blockIdx.x, gridDim.x, p.remap);
    const int bh = lb / p.slices, m0 = (lb % p.slices) * VS;
    const int T = p.T, NC = p.NC;
    const int64_t seq0 = static_cast<int64_t>(bh) * T;

    // global memory through buffer resources, one per tensor and sequence: reads past the
    // sequence's end return zero (flat gates, no keys, no values), writes past it are dropped
    constexpr int kRsrc = 0x00020000;
    auto rsrc = [](const void* base, int64_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrc);
    };

    if (NC == 0) {
        if (w < NV && p.s_out != nullptr) {
            float* so = p.s_out + (static_cast<int64_t>(bh) * DV + m0 + 16 * w + r16) * DK + 4 * g;
            const float* s0 = p.s0 ? p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * w + r16) * DK + 4 * g : nullptr;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) stf4(so + 16 * ct, s0 ? ldf4(s0 + 16 * ct) : zf4());
        }
        return;
    }

    if (w < 2) {
        // ================================================ chain waves
        // wave w carries S^T of value tiles vt = VW w .. VW w + VW - 1 (every key):
        // sacc[v][ct][e] = S[m0 + 16 vt + r16][chan(ct) + e]
        const bool live = w * VW < NV;
        f32x4 sacc[VW][KT];
#pragma unroll
        for (int v = 0; v < VW; ++v)
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                sacc[v][ct] = zf4();
                if (live && p.s0 != nullptr)
                    sacc[v][ct] = ldf4(p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * (VW * w + v) + r16) * DK + chan(ct));
            }
        const auto ro = rsrc(p.o + seq0 * DV, static_cast<int64_t>(T) * DV * 2);
        lds_barrier();   // the helpers' prologue
        for (int c = 0; c < NC; ++c) {
            if (live) {
                const u16* K = sK(c);
                const u16* Q = sQ(c);
                const float* E = sE(c);
                const u16* V = sV(c);
                const u16* P0 = sP(c, 0);
                const u16* P1 = sP(c, 1);
                // every LDS operand of the chunk is requested before the first product
                bf16x8 qa[CT][KB], pa[CT][JB], pc[CT][JB], kt[KT][JB];
                bf16x4 vv[VW][CT];
                f32x4 ed[KT];
#pragma unroll
                for (int it = 0; it < CT; ++it)
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        qa[it][kb] = *reinterpret_cast<const bf16x8*>(Q + TK::off(16 * it + r16, 32 * kb + 8 * g));
#pragma unroll
                for (int it = 0; it < CT; ++it) {
#pragma unroll
                    for (int v = 0; v < VW; ++v) vv[v][it] = tr_op_s<VS>(V, 16 * it, 16 * (VW * w + v), r16, g);
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
                        if (2 * jb > it) continue;
                        const bool hi = 2 * jb + 1 <= it;
                        const u16* r0 = P0 + (16 * it + r16) * RS + 32 * jb + 4 * g;
                        const u16* r1 = P1 + (16 * it + r16) * RS + 32 * jb + 4 * g;
                        pa[it][jb] = join8(ld4(r0), hi ? ld4(r0 + 16) : zero4());
                        pc[it][jb] = join8(ld4(r1), hi ? ld4(r1 + 16) : zero4());
                    }
                }
#pragma unroll
                for (int ct = 0; ct < KT; ++ct) {
                    ed[ct] = ldf4(E + chan(ct));
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
                        // A = (k 2^(B_last - B))^T: row r16 = key 32(ct / 2) + 8(r16 / 4) +
                        // 4(ct % 2) + r16 % 4, reduction slots = tokens 32jb + 4g + e and
                        // 32jb + 16 + 4g + e
                        const int col = 32 * (ct >> 1) + 8 * (r16 & 3) + 4 * (ct & 1);
                        kt[ct][jb] = join8(tr4(K + TK::off(32 * jb + 4 * g + (r16 >> 2), col)),
                                           tr4(K + TK::off(32 * jb + 16 + 4 * g + (r16 >> 2), col)));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);

#pragma unroll
                for (int v = 0; v < VW; ++v) {
                    bf16x8 sb[KB];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) sb[kb] = join8(cvt4(sacc[v][2 * kb]), cvt4(sacc[v][2 * kb + 1]));
                    // o^T = S_in (Q 2^B)^T: ot[it][e] = o[16it + r16][value 4g + e]
                    f32x4 ot[CT];
#pragma unroll
                    for (int it = 0; it < CT; ++it) ot[it] = zf4();
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int it = 0; it < CT; ++it) ot[it] = mfma_16x16x32(sb[kb], qa[it][kb], ot[it]);
                    bf16x8 vb[JB];
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) vb[jb] = join8(vv[v][2 * jb], vv[v][2 * jb + 1]);
                    // carry S^T <- diag(2^B_last) S^T + (K 2^(B_last - B))^T V, and o^T += V^T P^T
                    // with P the sum of the two helpers' partial triangles
#pragma unroll
                    for (int ct = 0; ct < KT; ++ct) sacc[v][ct] = sacc[v][ct] * ed[ct];
#pragma unroll
                    for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
                        for (int ct = 0; ct < KT; ++ct) sacc[v][ct] = mfma_16x16x32(kt[ct][jb], vb[jb], sacc[v][ct]);
#pragma unroll
                        for (int it = 0; it < CT; ++it) {
                            if (2 * jb > it) continue;
                            ot[it] = mfma_16x16x32(vb[jb], pa[it][jb], ot[it]);
                            ot[it] = mfma_16x16x32(vb[jb], pc[it][jb], ot[it]);
                        }
                    }
                    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
                    for (int it = 0; it < CT; ++it)
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, cvt4(ot[it])), ro,
                                                              ((c * C + 16 * it + r16) * DV + m0 + 16 * (VW * w + v) + 4 * g) * 2,
                                                              0, 0);
                }
            }
            lds_barrier();
        }
        if (live && p.s_out != nullptr) {
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                float* so = p.s_out + (static_cast<int64_t>(bh) * DV + m0 + 16 * (VW * w + v) + r16) * DK;
#pragma unroll
                for (int ct = 0; ct < KT; ++ct) stf4(so + chan(ct), sacc[v][ct]);
            }
        }
        return;
    }

    // ================================================ helper waves
    // helper hw: key channels key0 + e (e < KPL) of token tile g, tokens 16g + i (i < 16)
    const int ht = tid - 128;
    const int hw = w - 2;
    const int key0 = hw * HALF + KPL * r16;
    const auto rk = rsrc(p.k + seq0 * DK, static_cast<int64_t>(T) * DK * 2);
    const auto rq = rsrc(p.q + seq0 * DK, static_cast<int64_t>(T) * DK * 2);
    const auto rg = rsrc(p.alpha + seq0 * DK, static_cast<int64_t>(T) * DK * 4);
    const auto rv = rsrc(p.v + seq0 * DV, static_cast<int64_t>(T) * DV * 2);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

    // the register ring: a chunk's q, k, raw gates (this lane's keys and tokens) and v pieces
    struct Entry {
        unsigned q[16][QD], k[16][QD];
        float a[16][KPL];
        u32x4 v[NVP];
    };
    Entry ring[2];
    auto load = [&](Entry& e, int a) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = a * C + 16 * g + i;
            const int qo = (t * DK + key0) * 2, go = (t * DK + key0) * 4;
            if constexpr (KPL == 4) {
                const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rq, qo, 0, 0);
                const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(rk, qo, 0, 0);
                const f32x4 z = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, go, 0, 0));
                e.q[i][0] = x[0]; e.q[i][1] = x[1];
                e.k[i][0] = y[0]; e.k[i][1] = y[1];
#pragma unroll
                for (int j = 0; j < 4; ++j) e.a[i][j] = z[j];
            } else if constexpr (KPL == 2) {
                e.q[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rq, qo, 0, 0);
                e.k[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, qo, 0, 0);
                // (the whole vector cast: a bit cast of one element of a vector reads element 0)
                typedef float f32x2 __attribute__((ext_vector_type(2)));
                const f32x2 z = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, go, 0, 0));
                e.a[i][0] = z[0];
                e.a[i][1] = z[1];
            } else {
                e.q[i][0] = __builtin_amdgcn_raw_buffer_load_b16(rq, qo, 0, 0);
                e.k[i][0] = __builtin_amdgcn_raw_buffer_load_b16(rk, qo, 0, 0);
                e.a[i][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, go, 0, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < NVP; ++i) {
            const int pc = (ht + i * NH) % PV, j = pc / (VS / 8), col = (pc % (VS / 8)) * 8;
            e.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((a * C + j) * DV + m0 + col) * 2, 0, 0);
        }
    };
    // a lane's KPL bf16 values to LDS
    auto put = [&](u16* dst, const float* x) __attribute__((always_inline)) {
        if constexpr (KPL == 4) {
            f32x4 y = {x[0], x[1], x[2], x[3]};
            st4(dst, cvt4(y));
        } else if constexpr (KPL == 2) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            bf16x2 y;
            y[0] = static_cast<__bf16>(x[0]);
            y[1] = static_cast<__bf16>(x[1]);
            *reinterpret_cast<bf16x2*>(dst) = y;
        } else {
            *dst = f32_to_bf16_bits(x[0]);
        }
    };
    // chunk a's gates and operands into slot a: the scan, the tile references, the four
    // rescaled copies of q and k, the F table, 2^B_last and the v slice
    auto prepare = [&](const Entry& e, int a) __attribute__((always_inline)) {
        float tot[KPL], inc[KPL], off[KPL], mr[KPL], rq2[KPL], wk2[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) s += e.a[i][j] * kLog2e;
            tot[j] = s;
            inc[j] = s;
        }
        // inclusive scan of the tile totals over the four tiles (lane groups)
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const float y = __shfl_up(inc[j], 16, 64);
            if (g >= 1) inc[j] += y;
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const float y = __shfl_up(inc[j], 32, 64);
            if (g >= 2) inc[j] += y;
        }
        float* E = sE(a);
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const float pre = inc[j] - tot[j];                   // B just before the tile
            const float bl = __shfl(inc[j], 48 + r16, 64);      // B_last
            mr[j] = tile_ref(pre, inc[j]);
            off[j] = pre - mr[j];
            rq2[j] = ex2(mr[j]);
            wk2[j] = ex2(bl - mr[j]);
            if (g == 0) E[key0 + j] = ex2(bl);
        }
        u16* Qt = sQ(a);
        u16* Kt = sK(a);
        float run[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) run[j] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float qh[KPL], kh[KPL], qt[KPL], kt[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                run[j] += e.a[i][j] * kLog2e;
                const float d = run[j] + off[j];   // B - m
                const float qv = bf_at(e.q[i][j >> 1], j & 1), kv = bf_at(e.k[i][j >> 1], j & 1);
                qh[j] = qv * ex2(d);
                kh[j] = kv * ex2(-d);
                qt[j] = qh[j] * rq2[j];
                kt[j] = kh[j] * wk2[j];
            }
            const int o = TK::off(16 * g + i, key0);
            put(sQh + o, qh);
            put(sKh + o, kh);
            put(Qt + o, qt);
            put(Kt + o, kt);
        }
        // F[pair (it, jt)][key] = 2^(m_it - m_jt), jt < it, pairs in row order
        float* F = reinterpret_cast<float*>(smem + Lay::oF + hw * Lay::FBUF);
#pragma unroll
        for (int jt = 0; jt < CT - 1; ++jt)
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const float mj = __shfl(mr[j], 16 * jt + r16, 64);
                if (g > jt) F[((g * (g - 1)) / 2 + jt) * HALF + KPL * r16 + j] = ex2(mr[j] - mj);
            }
        u16* Vs = sV(a);
#pragma unroll
        for (int i = 0; i < NVP; ++i) {
            const int pc = ht + i * NH;
            if (PV % NH == 0 || pc < PV) {
                const int j = pc / (VS / 8), col = (pc % (VS / 8)) * 8;
                *reinterpret_cast<u32x4*>(Vs + TV::off(j, col)) = e.v[i];
            }
        }
    };
    // this helper's partial triangle of chunk a over its key half: P[i][j] for j <= i (tile
    // pairs below the diagonal through F), bf16, into its slot
    auto triangle = [&](int a) __attribute__((always_inline)) {
        const float* F = reinterpret_cast<const float*>(smem + Lay::oF + hw * Lay::FBUF);
        u16* PP = sP(a, hw);
        bf16x8 qh[CT][KBH], kh[CT][KBH];
#pragma unroll
        for (int it = 0; it < CT; ++it)
#pragma unroll
            for (int kb = 0; kb < KBH; ++kb) {
                const int lc = 8 * (kb + KBH * g);   // key within the half
                qh[it][kb] = as_bf16x8(u16x8{0, 0, 0, 0, 0, 0, 0, 0});
                kh[it][kb] = qh[it][kb];
                if (lc < HALF) {
                    qh[it][kb] = *reinterpret_cast<const bf16x8*>(sQh + TK::off(16 * it + r16, hw * HALF + lc));
                    kh[it][kb] = *reinterpret_cast<const bf16x8*>(sKh + TK::off(16 * it + r16, hw * HALF + lc));
                }
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < CT; ++it) {
            const int i = 16 * it + r16;
#pragma unroll
            for (int jt = 0; jt <= it; ++jt) {
                f32x4 acc = zf4();
#pragma unroll
                for (int kb = 0; kb < KBH; ++kb) {
                    bf16x8 qb = qh[it][kb];
                    const int lc = 8 * (kb + KBH * g);
                    if (jt < it && lc < HALF) {
                        const float* f = F + ((it * (it - 1)) / 2 + jt) * HALF + lc;
                        const f32x4 f0 = ldf4(f), f1 = ldf4(f + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            qb[e] = static_cast<__bf16>(static_cast<float>(qb[e]) * f0[e]);
                            qb[4 + e] = static_cast<__bf16>(static_cast<float>(qb[4 + e]) * f1[e]);
                        }
                    }
                    acc = mfma_16x16x32(kh[jt][kb], qb, acc);
                }
                // acc[e] = partial P[i][j], j = 16jt + 4g + e
                if (jt == it) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * g + e > r16) acc[e] = 0.f;
                }
                st4(PP + i * RS + 16 * jt + 4 * g, cvt4(acc));
            }
        }
    };

    // prologue: chunk 0 prepared and its triangles formed, chunk 1 in flight
    const int last = NC - 1;
    load(ring[0], 0);
    load(ring[1], last > 0 ? 1 : 0);
    prepare(ring[0], 0);
    load(ring[0], last > 1 ? 2 : last);
    triangle(0);
    lds_barrier();
    // step c: chunk c + 1 from ring slot R into LDS slot c + 1 and its triangles, then the
    // loads of chunk c + 3 into R (past the end they are clamped to the last chunk and unused)
    auto step = [&](int c, auto slot) __attribute__((always_inline)) {
        constexpr int R = decltype(slot)::value;
        if (c + 1 < NC) {
            prepare(ring[R], c + 1);
            load(ring[R], c + 3 < NC ? c + 3 : last);
            triangle(c + 1);
        }
        lds_barrier();
    };
    int c = 0;
    for (; c + 1 < NC; c += 2) {
        step(c, std::integral_constant<int, 1>{});
        step(c + 1, std::integral_constant<int, 0>{});
    }
    if (c < NC) step(c, std::integral_constant<int, 1>{});
}

// ====================================================================== launch
// Slices of 64 value channels (two chain waves of two value tiles) when that still gives
// every CU a workgroup, else 32, else 16.
template <int DK, int DV, int VS, int VW>
hipError_t launch_gla_sp_vs(const ChunkArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    GspParams p{};
    p.q = static_cast<const u16*>(a.q);
    p.k = static_cast<const u16*>(a.k);
    p.v = static_cast<const u16*>(a.v);
    p.alpha = a.gate;
    p.s0 = a.s0;
    p.o = static_cast<u16*>(a.o);
    p.s_out = a.s_out;
    p.T = a.T;
    p.NC = (a.T + 63) / 64;
    p.slices = DV / VS;
    const int64_t grid = heads * p.slices;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((gla_sp_kernel<DK, DV, VS, VW>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_gla_sp_dv(const ChunkArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if constexpr (DV >= 64) {
        if (heads * (DV / 64) >= kCUs) return launch_gla_sp_vs<DK, DV, 64, 2>(a, stream);
    }
    if constexpr (DV >= 32) {
        if (heads * (DV / 32) >= kCUs) return launch_gla_sp_vs<DK, DV, 32, 1>(a, stream);
    }
    return launch_gla_sp_vs<DK, DV, 16, 1>(a, stream);
}

inline hipError_t launch_gla_sp(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk * 1000 + a.dv) {
        case 32016: return launch_gla_sp_dv<32, 16>(a, stream);
        case 32032: return launch_gla_sp_dv<32, 32>(a, stream);
        case 32064: return launch_gla_sp_dv<32, 64>(a, stream);
        case 32128: return launch_gla_sp_dv<32, 128>(a, stream);
        case 64016: return launch_gla_sp_dv<64, 16>(a, stream);
        case 64032: return launch_gla_sp_dv<64, 32>(a, stream);
        case 64064: return launch_gla_sp_dv<64, 64>(a, stream);
        case 64128: return launch_gla_sp_dv<64, 128>(a, stream);
        case 128016: return launch_gla_sp_dv<128, 16>(a, stream);
        case 128032: return launch_gla_sp_dv<128, 32>(a, stream);
        case 128064: return launch_gla_sp_dv<128, 64>(a, stream);
        case 128128: return launch_gla_sp_dv<128, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace ck
}  // namespace glr
