// GLA's chunked forward in one pass (bf16 storage, chunk 64, d_k of 64 or 128).
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
// One workgroup of eight waves per (sequence, value slice of VS channels), one barrier per
// chunk. Chain waves 0 .. 3 each hold S^T of one 16-channel value tile in fp32 MFMA
// accumulators across the chunks; helper waves 4 .. 7 make the next chunk's operands while
// the chain works on the current one, so each SIMD runs one chain wave and one helper wave
// (the chain's LDS and MFMA waits and the helpers' VALU work overlap):
//   - helper h owns key channels [h d_k / 4, (h + 1) d_k / 4); lane (tq, kq) loads d_k / 16
//     of them for the four tokens 4tq .. 4tq + 3 (16-byte pieces of q and k at d_k = 128). A
//     DPP row of 16 lanes then holds one key group's 64 tokens: the scan of the gates runs
//     along the row, its lane quads are the 16-token tiles;
//   - per token tile and key, the reference m is the cumulative gate just before the tile,
//     lowered to 80 nats above the tile's last one when the tile decays more than that, so
//     that q 2^(B - m) and k 2^(m - B) stay finite for tiles down to -160 nats. The chain's
//     operands follow from them by one factor each: q 2^B = (q 2^(B - m)) 2^m and
//     k 2^(B_last - B) = (k 2^(m - B)) 2^(B_last - m), both at most |q| and |k|;
//   - when every cumulative gate of a chunk is within 2^+-100 (a bound each helper publishes
//     two steps ahead, so that all waves agree), the reference is the chunk's start: the
//     triangle then takes q 2^B and k 2^-B, and the carry k 2^-B with 2^B_last applied after
//     the sum, so the helpers write two rescaled copies instead of four and no F table;
//   - each chain wave forms the whole causal triangle itself (ten 16 x 16 tile pairs over all
//     keys, pairs below the diagonal joined by F = 2^(m_it - m_jt) <= 1 on the q operand): a
//     pair's accumulator is, lane for lane, the half of P V's B operand it feeds, so P stays
//     in registers and the helpers only prepare.
// The chain's work per chunk is that of the scalar decay with the decay of S^T taken per key
// (one factor per accumulator) and the token weights already inside the operands.
//
// LDS (d_k 128, 64-channel slices), every buffer in two slots: the four rescaled copies of q
// and k, 2^B_last, the F table and the v slice, 151 KB. Buffer offsets are 31-bit: one
// sequence's raw gates (rows padded to whole chunks times d_k times 4 bytes), q, k, v and o
// must stay below 2^31 bytes.
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

// The swizzled tile of q and k rows with its phase also turned by bits 4-5 of the row: a
// helper's store of rows 4tq + s over the sixteen tq of a DPP row then lands on sixteen
// different 16-byte bank groups (d_k 128; two to a group at d_k 64, four with the plain tile),
// while every access within one 16-row block (the chain's and the triangle's reads) sees the
// plain tile's pattern.
template <int W>
struct GlaTile {
    static_assert(W == 64 || W == 128, "rows of 64 or 128 keys");
    static constexpr int STRIDE = W;
    __device__ static __forceinline__ int off(int r, int c) {
        const int h = (W == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1))) ^
                      (((r >> 4) & 3) << 1);
        return r * W + ((((c >> 3) ^ h) << 3) | (c & 7));
    }
};

template <int DK, int VS>
struct GspLayout {
    static constexpr int C = 64;
    using TK = GlaTile<DK>;     // q and k rows (and their rescaled forms)
    using TV = SwzTile<VS>;     // the v slice
    static constexpr int al(int x) { return (x + 15) / 16 * 16; }
    static constexpr int KBUF = al(C * TK::STRIDE * 2);
    static constexpr int VBUF = al(C * TV::STRIDE * 2);
    static constexpr int EBUF = al(DK * 4);
    static constexpr int FBUF = al(6 * DK * 4);
    static constexpr int oK = 0;                 // k 2^(B_last - B): the carry's (chunks that are not flat)
    static constexpr int oQ = oK + 2 * KBUF;     // q 2^B: the readout's
    static constexpr int oKh = oQ + 2 * KBUF;    // k 2^(m - B): the triangle's
    static constexpr int oQh = oKh + 2 * KBUF;   // q 2^(B - m): the triangle's (chunks that are not flat)
    static constexpr int oE = oQh + 2 * KBUF;    // 2^B_last per key
    static constexpr int oF = oE + 2 * EBUF;     // F [pair][key] (chunks that are not flat)
    static constexpr int oV = oF + 2 * FBUF;     // the v slice
    static constexpr int oS = oV + 2 * VBUF;     // each helper's bound on a chunk's decay, four slots
    static constexpr int bytes = oS + 4 * 4 * 4;
    static_assert(bytes <= 160 * 1024, "LDS budget of the GLA single pass exceeded");
};

// bf16 element e (e < 2) of a packed pair, as float
__device__ __forceinline__ float bf_at(unsigned x, int e) {
    return __builtin_bit_cast(float, e ? (x & 0xffff0000u) : (x << 16));
}

template <int DK, int DV, int VS>
__global__ __launch_bounds__(512)
void gla_sp_kernel(GspParams p) {
    constexpr int C = 64;
    using Lay = GspLayout<DK, VS>;
    using TK = typename Lay::TK;
    using TV = typename Lay::TV;
    constexpr int NV = VS / 16;                 // value tiles: chain waves 0 .. NV - 1
    constexpr int CT = C / 16, JB = CT / 2;     // token tiles, 32-token blocks
    constexpr int KT = DK / 16, KB = DK / 32;   // key tiles, 32-key blocks
    constexpr int QPH = DK / 4;                 // keys per helper
    constexpr int KPL = DK / 16;                // keys per helper lane (four tokens each)
    constexpr int NH = 256;                     // helper threads
    constexpr int PV = C * VS / 8, NVP = (PV + NH - 1) / NH;
    static_assert(DK == 64 || DK == 128, "d_k of 64 or 128");
    static_assert(DV % VS == 0 && (VS == 16 || VS == 32 || VS == 64), "value slices of 16, 32 or 64 channels");

    __shared__ __align__(16) unsigned char smem[Lay::bytes];
    auto sK = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oK + (b & 1) * Lay::KBUF); };
    auto sQ = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oQ + (b & 1) * Lay::KBUF); };
    auto sKh = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oKh + (b & 1) * Lay::KBUF); };
    auto sQh = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oQh + (b & 1) * Lay::KBUF); };
    auto sE = [&](int b) { return reinterpret_cast<float*>(smem + Lay::oE + (b & 1) * Lay::EBUF); };
    auto sF = [&](int b) { return reinterpret_cast<float*>(smem + Lay::oF + (b & 1) * Lay::FBUF); };
    auto sV = [&](int b) { return reinterpret_cast<u16*>(smem + Lay::oV + (b & 1) * Lay::VBUF); };
    float* const sB = reinterpret_cast<float*>(smem + Lay::oS);

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
    // chunk a is flat when every cumulative gate in it is within 2^+-100 (the largest of the
    // four helpers' bounds, published two steps ahead in slot a mod 4): the triangle then takes
    // q 2^B and k 2^-B with no tile references, and the carry k 2^-B with 2^B_last applied to
    // the sum. Every wave reads the same slot, so all take the same form.
    auto flat_chunk = [&](int a) __attribute__((always_inline)) {
        const float* b = sB + 4 * (a & 3);
        return __builtin_amdgcn_readfirstlane(fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])) <= 100.f ? 1 : 0) != 0;
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

    if (w < 4) {
        // ================================================ chain waves
        // wave w < NV carries S^T of value tile w (every key):
        // sacc[ct][e] = S[m0 + 16w + r16][chan(ct) + e]
        const bool live = w < NV;
        f32x4 sacc[KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            sacc[ct] = zf4();
            if (live && p.s0 != nullptr)
                sacc[ct] = ldf4(p.s0 + (static_cast<int64_t>(bh) * DV + m0 + 16 * w + r16) * DK + chan(ct));
        }
        const auto ro = rsrc(p.o + seq0 * DV, static_cast<int64_t>(T) * DV * 2);
        // one chunk: the readout S_in (Q 2^B)^T, the causal triangle (formed here, in the
        // registers P V reads it from), P V, the store of o and the carry of S^T
        auto step = [&](int c, auto flat_c) __attribute__((always_inline)) {
            constexpr bool FL = decltype(flat_c)::value;
            const u16* Q = sQ(c);
            const u16* Kh = sKh(c);
            const float* E = sE(c);
            const u16* V = sV(c);
            // o^T = S_in (Q 2^B)^T + V^T P^T: ot[it][e] = o[16it + r16][value 16w + 4g + e]
            bf16x8 qa[CT][KB], vb[JB];
            f32x4 ot[CT];
            auto readout = [&]() __attribute__((always_inline)) {
                bf16x8 sb[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sb[kb] = join8(cvt4(sacc[2 * kb]), cvt4(sacc[2 * kb + 1]));
#pragma unroll
                for (int it = 0; it < CT; ++it)
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        qa[it][kb] = *reinterpret_cast<const bf16x8*>(Q + TK::off(16 * it + r16, 32 * kb + 8 * g));
#pragma unroll
                for (int it = 0; it < CT; ++it) {
                    ot[it] = zf4();
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) ot[it] = mfma_16x16x32(sb[kb], qa[it][kb], ot[it]);
                }
            };
            // the triangle: tile pair (it, jt <= it) accumulates P[16it + r16][16jt + 4g + e],
            // which is the half of P V's B operand for tokens 16jt + 4g + e
            bf16x4 ph[CT][CT];
            if constexpr (FL) {
                // q 2^B (the readout's operand) against k 2^-B, one key-row tile jt at a time
                readout();
#pragma unroll
                for (int jt = 0; jt < CT; ++jt) {
                    bf16x8 kr[KB];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        kr[kb] = *reinterpret_cast<const bf16x8*>(Kh + TK::off(16 * jt + r16, 32 * kb + 8 * g));
#pragma unroll
                    for (int it = jt; it < CT; ++it) {
                        f32x4 acc = zf4();
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) acc = mfma_16x16x32(kr[kb], qa[it][kb], acc);
                        if (jt == it) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (4 * g + e > r16) acc[e] = 0.f;
                        }
                        ph[it][jt] = cvt4(acc);
                    }
                }
            } else {
                // q 2^(B - m) against k 2^(m - B) with the tile references m, one query tile at
                // a time, pairs below the diagonal joined by F on q; the readout after it
                const u16* Qh = sQh(c);
                const float* Fc = sF(c);
#pragma unroll
                for (int it = 0; it < CT; ++it) {
                    bf16x8 qh[KB];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        qh[kb] = *reinterpret_cast<const bf16x8*>(Qh + TK::off(16 * it + r16, 32 * kb + 8 * g));
#pragma unroll
                    for (int jt = 0; jt <= it; ++jt) {
                        f32x4 acc = zf4();
#pragma unroll
                        for (int kb = 0; kb < KB; ++kb) {
                            const bf16x8 kr = *reinterpret_cast<const bf16x8*>(Kh + TK::off(16 * jt + r16, 32 * kb + 8 * g));
                            bf16x8 qb = qh[kb];
                            if (jt < it) {
                                const float* f = Fc + ((it * (it - 1)) / 2 + jt) * DK + 32 * kb + 8 * g;
                                const f32x4 f0 = ldf4(f), f1 = ldf4(f + 4);
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    qb[e] = static_cast<__bf16>(static_cast<float>(qb[e]) * f0[e]);
                                    qb[4 + e] = static_cast<__bf16>(static_cast<float>(qb[4 + e]) * f1[e]);
                                }
                            }
                            acc = mfma_16x16x32(kr, qb, acc);
                        }
                        if (jt == it) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (4 * g + e > r16) acc[e] = 0.f;
                        }
                        ph[it][jt] = cvt4(acc);
                        // one pair's k rows and F at a time
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
                readout();
            }
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
                vb[jb] = join8(tr_op_s<VS>(V, 32 * jb, 16 * w, r16, g), tr_op_s<VS>(V, 32 * jb + 16, 16 * w, r16, g));
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                for (int it = 0; it < CT; ++it)
                    if (2 * jb <= it)
                        ot[it] = mfma_16x16x32(vb[jb], join8(ph[it][2 * jb], 2 * jb + 1 <= it ? ph[it][2 * jb + 1] : zero4()), ot[it]);
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int it = 0; it < CT; ++it)
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, cvt4(ot[it])), ro,
                                                      ((c * C + 16 * it + r16) * DV + m0 + 16 * w + 4 * g) * 2, 0, 0);
            // carry: S^T <- diag(2^B_last) S^T + (K 2^(B_last - B))^T V, or for a flat chunk
            // S^T <- diag(2^B_last) (S^T + (K 2^-B)^T V)
            const u16* KC = FL ? Kh : sK(c);
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) {
                // A = (k 2^(B_last - B))^T: row r16 = key 32(ct / 2) + 8(r16 / 4) + 4(ct % 2) +
                // r16 % 4, reduction slots = tokens 32jb + 4g + e and 32jb + 16 + 4g + e
                const int col = 32 * (ct >> 1) + 8 * (r16 & 3) + 4 * (ct & 1);
                const f32x4 el = ldf4(E + chan(ct));
                f32x4 a = FL ? sacc[ct] : sacc[ct] * el;
#pragma unroll
                for (int jb = 0; jb < JB; ++jb)
                    a = mfma_16x16x32(join8(tr4(KC + TK::off(32 * jb + 4 * g + (r16 >> 2), col)),
                                            tr4(KC + TK::off(32 * jb + 16 + 4 * g + (r16 >> 2), col))),
                                      vb[jb], a);
                sacc[ct] = FL ? a * el : a;
            }
        };
        lds_barrier();   // the helpers' prologue: chunk 0's decay bound, then chunk 0
        lds_barrier();
        for (int c = 0; c < NC; ++c) {
            if (live) {
                if (flat_chunk(c))
                    step(c, std::true_type{});
                else
                    step(c, std::false_type{});
            }
            lds_barrier();   // chunk c + 1 ready; slot c free
        }
        if (live && p.s_out != nullptr) {
            float* so = p.s_out + (static_cast<int64_t>(bh) * DV + m0 + 16 * w + r16) * DK;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) stf4(so + chan(ct), sacc[ct]);
        }
        return;
    }

    // ================================================ helper waves
    // helper hw owns key channels [hw d_k / 4, (hw + 1) d_k / 4); lane (tq = lane & 15,
    // kq = lane >> 4) holds KPL = d_k / 16 of them, key0 + e, for the four tokens 4tq + s of
    // each chunk (16-byte loads of q and k at d_k = 128). So a DPP row of 16 lanes holds one
    // key group's 64 tokens, and its lane quads 4it .. 4it + 3 token tile it: the scan of the
    // gates runs along the row, the tile references come by quad broadcasts and the joins F by
    // row shifts.
    const int ht = tid - 256;
    const int hw = w - 4;
    const int tq = lane & 15, kq = lane >> 4;
    const int key0 = hw * QPH + KPL * kq;
    const auto rk = rsrc(p.k + seq0 * DK, static_cast<int64_t>(T) * DK * 2);
    const auto rq = rsrc(p.q + seq0 * DK, static_cast<int64_t>(T) * DK * 2);
    const auto rg = rsrc(p.alpha + seq0 * DK, static_cast<int64_t>(T) * DK * 4);
    const auto rv = rsrc(p.v + seq0 * DV, static_cast<int64_t>(T) * DV * 2);
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int QW = KPL / 2;    // 32-bit words of a lane's q or k piece of one token

    // the register ring: a chunk's q, k, raw gates (this lane's keys and tokens) and v pieces
    struct Entry {
        unsigned q[4][QW], k[4][QW];
        float a[4][KPL];
        u32x4 v[NVP];
    };
    Entry ring;
    // token 4tq + s of chunk a (one base offset per chunk; the token's part is a constant the
    // loads take as their immediate offset)
    auto load_qk = [&](Entry& e, int a, int s) __attribute__((always_inline)) {
        const int qo = ((a * C + 4 * tq) * DK + key0) * 2 + s * DK * 2;
        if constexpr (KPL == 8) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, qo, 0, 0);
            const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(rk, qo, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e.q[s][j] = x[j];
                e.k[s][j] = y[j];
            }
        } else {
            const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rq, qo, 0, 0);
            const u32x2 y = __builtin_amdgcn_raw_buffer_load_b64(rk, qo, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                e.q[s][j] = x[j];
                e.k[s][j] = y[j];
            }
        }
    };
    auto load_gates = [&](Entry& e, int a, int s) __attribute__((always_inline)) {
        const int go = ((a * C + 4 * tq) * DK + key0) * 4 + s * DK * 4;
#pragma unroll
        for (int h = 0; h < KPL / 4; ++h) {
            // (the whole vector cast: a bit cast of one element of a vector reads element 0)
            const f32x4 z = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, go + 16 * h, 0, 0));
#pragma unroll
            for (int j = 0; j < 4; ++j) e.a[s][4 * h + j] = z[j];
        }
    };
    auto load_v = [&](Entry& e, int a) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NVP; ++i) {
            const int pc = (ht + i * NH) % PV, j = pc / (VS / 8), col = (pc % (VS / 8)) * 8;
            e.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, ((a * C + j) * DV + m0 + col) * 2, 0, 0);
        }
    };
    // a lane's KPL bf16 values to LDS (16 or 8 bytes)
    auto put = [&](u16* dst, const float* x) __attribute__((always_inline)) {
        if constexpr (KPL == 8) {
            *reinterpret_cast<bf16x8*>(dst) = pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
        } else {
            f32x4 y = {x[0], x[1], x[2], x[3]};
            st4(dst, cvt4(y));
        }
    };
    // an upper bound on |B| over chunk a (log2 units; the sum over its tokens of the largest
    // |log alpha| among a lane's keys, along the row, the largest of the four rows), published
    // per helper in slot a mod 4, two steps before the chain reads it
    auto bound = [&](const Entry& e, int a) __attribute__((always_inline)) {
        float sm = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            float mx = 0.f;
#pragma unroll
            for (int j = 0; j < KPL; ++j) mx = fmaxf(mx, fabsf(e.a[s2][j]));
            sm += mx;
        }
        sm = row16_sum(sm);
        auto rl = [&](int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sm), l)); };
        const float b = fmaxf(fmaxf(rl(0), rl(16)), fmaxf(rl(32), rl(48))) * kLog2e;
        if (lane == 0) sB[4 * (a & 3) + hw] = b;
    };
    // chunk a's gates and operands into slot a: the scan, the tile references, the rescaled
    // copies of q and k (four; two when the chunk is flat), the F table (not when flat),
    // 2^B_last and the v slice. The ring's registers are refilled with chunk nx as soon as they
    // are used, so the next chunk's loads overlap the rest of this step and the next one's
    // start. The refill is unconditional (the last step reloads a chunk that is not used): with
    // the same loads on every path, each wait for a ring register counts only the loads issued
    // before it, not those of the next chunk.
    auto prepare = [&](Entry& e, int a, int nx, bool flat) __attribute__((always_inline)) {
        // running sums over the lane's four tokens (log2 units)
        float sr[4][KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            float r = 0.f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                r += e.a[s][j] * kLog2e;
                sr[s][j] = r;
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) load_gates(e, nx, s);
        // along the row: the cumulative gate before the lane's quad (ex), the tile's reference
        // m (from the gate before its first quad and after its last), B_last
        float off[KPL], mr[KPL], rq2[KPL], wk2[KPL], el[KPL];
        // the scan (y, along the row) and the row sum (b, B_last) stage by stage over every key,
        // so that the keys' DPP chains interleave
        float y[KPL], b[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) y[j] = b[j] = sr[3][j];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            y[j] += dpp_move<0x111>(y[j]);   // row_shr:1 (lanes shifted in from outside the row read 0)
            b[j] += dpp_move<0xB1>(b[j]);    // quad_perm [1,0,3,2]
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            y[j] += dpp_move<0x112>(y[j]);   // row_shr:2
            b[j] += dpp_move<0x4E>(b[j]);    // quad_perm [2,3,0,1]
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            y[j] += dpp_move<0x114>(y[j]);   // row_shr:4
            b[j] += dpp_move<0x141>(b[j]);   // row_half_mirror
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            y[j] += dpp_move<0x118>(y[j]);   // row_shr:8
            b[j] += dpp_move<0x140>(b[j]);   // row_mirror
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
            const float ex = y[j] - sr[3][j];
            const float pre = dpp_move<0x00>(ex);      // quad_perm [0,0,0,0]: before the tile
            const float tend = dpp_move<0xFF>(y[j]);   // quad_perm [3,3,3,3]: its last token
            mr[j] = flat ? 0.f : tile_ref(pre, tend);
            off[j] = ex - mr[j];
            rq2[j] = ex2(mr[j]);
            wk2[j] = ex2(b[j] - mr[j]);
            el[j] = ex2(b[j]);
        }
        // (one store after the scan of every key: a store per key would split the keys' scans)
        if (tq == 0) {
            float* E = sE(a) + key0;
#pragma unroll
            for (int h = 0; h < KPL / 4; ++h) {
                f32x4 y = {el[4 * h], el[4 * h + 1], el[4 * h + 2], el[4 * h + 3]};
                stf4(E + 4 * h, y);
            }
        }
        u16* Qt = sQ(a);
        u16* Kt = sK(a);
        u16* Qh = sQh(a);
        u16* Kh = sKh(a);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float qh[KPL], kh[KPL], qv[KPL], kv[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const float d = sr[s][j] + off[j];   // B - m
                const float x = bf_at(e.q[s][j >> 1], j & 1), y = bf_at(e.k[s][j >> 1], j & 1);
                qh[j] = x * ex2(d);
                kh[j] = y * ex2(-d);
                qv[j] = qh[j] * rq2[j];
                kv[j] = kh[j] * wk2[j];
            }
            const int o = TK::off(4 * tq + s, key0);
            if (!flat) {
                put(Qh + o, qh);
                put(Kt + o, kv);
            }
            put(Kh + o, kh);
            put(Qt + o, qv);
            __builtin_amdgcn_sched_barrier(0);
            load_qk(e, nx, s);
        }
        // F[pair (it, jt)][key] = 2^(m_it - m_jt), jt < it, pairs in row order: m_jt from the
        // quad 4(it - jt) lanes down the row, written by the tile's first lane
        const int it = tq >> 2;
        float* const Fa = sF(a);
#pragma unroll
        for (int dl = 1; dl < CT; ++dl) {
            if (flat) break;
            float f[KPL];
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const float mj = dl == 1 ? dpp_move<0x114>(mr[j]) : dl == 2 ? dpp_move<0x118>(mr[j]) : dpp_move<0x11C>(mr[j]);
                f[j] = ex2(mr[j] - mj);
            }
            if ((tq & 3) == 0 && it >= dl) {
                float* dst = Fa + ((it * (it - 1)) / 2 + it - dl) * DK + key0;
#pragma unroll
                for (int h = 0; h < KPL / 4; ++h) {
                    f32x4 y = {f[4 * h], f[4 * h + 1], f[4 * h + 2], f[4 * h + 3]};
                    stf4(dst + 4 * h, y);
                }
            }
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
        load_v(e, nx);
    };

    // prologue: chunk 0's decay bound; chunk 0 prepared (chunk 1 requested behind it) and
    // chunk 1's bound
    const int last = NC - 1;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        load_qk(ring, 0, s);
        load_gates(ring, 0, s);
    }
    load_v(ring, 0);
    bound(ring, 0);
    lds_barrier();
    prepare(ring, 0, last > 0 ? 1 : 0, flat_chunk(0));
    if (last > 0) bound(ring, 1);
    lds_barrier();
    // step c (the chain on chunk c): chunk c + 1 into slot c + 1 (chunk c + 2 requested behind
    // it), then chunk c + 2's bound
    for (int c = 0; c < NC; ++c) {
        if (c + 1 < NC) prepare(ring, c + 1, c + 2 < NC ? c + 2 : last, flat_chunk(c + 1));
        if (c + 2 < NC) bound(ring, c + 2);
        lds_barrier();
    }
}

// ====================================================================== launch
// Slices of 64 value channels (four chain waves) when that still gives every CU a workgroup,
// else 32, else 16.
template <int DK, int DV, int VS>
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
    hipLaunchKernelGGL((gla_sp_kernel<DK, DV, VS>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_gla_sp_dv(const ChunkArgs& a, hipStream_t stream) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if constexpr (DV >= 64) {
        if (heads * (DV / 64) >= kCUs) return launch_gla_sp_vs<DK, DV, 64>(a, stream);
    }
    if constexpr (DV >= 32) {
        if (heads * (DV / 32) >= kCUs) return launch_gla_sp_vs<DK, DV, 32>(a, stream);
    }
    return launch_gla_sp_vs<DK, DV, 16>(a, stream);
}

inline hipError_t launch_gla_sp(const ChunkArgs& a, hipStream_t stream) {
    switch (a.dk * 1000 + a.dv) {
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
