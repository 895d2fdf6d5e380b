/*
 * glr.h - C ABI of the gated linear recurrences library (gfx950 / MI355X).
 *
 * The library evaluates the causal linear-attention recurrence
 *     S_t = S_{t-1} G_t + (write of token t),   o_t = S_t q_t
 * on a fixed-size memory S of shape [d_v, d_k] (rows = value channels,
 * columns = key channels), for the gate variants fixed by the book chapter
 * "Scrivere meglio nella memoria: gate e delta rule" (transition table of the
 * section "Le ricorrenze come regressione online") and evaluated in the
 * chunkwise form of "Le architetture lineari: RetNet, RWKV, xLSTM" (section
 * "RetNet: la retention e le sue tre forme", Fig. 16.5): a masked decay
 * triangle inside each chunk of `chunk` tokens and the memory carried from one
 * chunk to the next. The readout of token t comes after its write.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers owned by the caller; the library allocates
 *    nothing, keeps no per-call state and may be called from several host
 *    threads on different streams.
 *  - Chunk entry points take a device `workspace` of `workspace_bytes` bytes,
 *    16-byte aligned, for data passed between their kernels: the one addition
 *    to plain (pointers, sizes, stream) signatures, since the library
 *    allocates nothing and data handed from one kernel of a call to the next
 *    must live in caller-owned memory.  Its size comes from
 *    la_chunk_workspace_size() and may be 0, in which case workspace may be
 *    NULL.  Its contents on entry do not matter and are undefined on exit.
 *    Two calls in flight at the same time need separate workspaces.
 *  - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued and
 *    the call returns without synchronising; outputs are valid once the stream
 *    has reached the enqueued work.
 *  - Layout (row-major, contiguous):  q, k [B][H][T][d_k];  v, o [B][H][T][d_v];
 *    states s0, s_out [B][H][d_v][d_k] float32.  Gates and write strengths are
 *    float32 whatever `dtype` is.
 *  - `dtype` is the storage type of q, k, v and o: LA_F32 (float32, fp32
 *    arithmetic throughout) or LA_BF16 (bfloat16 inputs and output, matrix
 *    products on bf16 MFMA with fp32 accumulation, fp32 memory).  The output is
 *    rounded to nearest-even when stored as bf16.
 *  - s0 == NULL starts from the zero memory; s_out == NULL skips storing the
 *    final memory.  s0 == s_out (in-place continuation) is allowed; o must not
 *    alias any input.
 *  - T may be any value >= 0; T % chunk != 0 leaves a shorter last chunk.  With
 *    T == 0 nothing is written to o and s_out receives s0 (or zeros).  B == 0
 *    or H == 0 is a no-op.
 *  - Every pointer that is read or written must be 16-byte aligned.
 *
 * Errors (no exception crosses the ABI):
 *  - LA_ERR_INVALID: a required pointer is NULL, a size is negative, a pointer
 *    is misaligned, chunk < 1, or the workspace is smaller than required;
 *    nothing is enqueued.
 *  - LA_ERR_UNSUPPORTED: d_k or d_v not in {16, 32, 64, 128}, chunk not in
 *    {16, 32, 64}, B * H >= 2^24 or B * H * ceil(T / chunk) >= 2^31; nothing
 *    is enqueued.
 *  - LA_ERR_HIP: a launch failed (the HIP error is kept in la_last_error()).
 *    Faults during execution surface at the caller's next synchronisation.
 *  NaN and Inf in the inputs propagate; they are not checked.
 */
#ifndef GLR_H
#define GLR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
    LA_OK = 0,
    LA_ERR_INVALID = 1,
    LA_ERR_UNSUPPORTED = 2,
    LA_ERR_HIP = 3
} la_status;

typedef enum la_dtype {
    LA_F32 = 0,
    LA_BF16 = 1
} la_dtype;

typedef enum la_fuse {
    LA_FUSE_QK_SILU_L2 = 1,    /* q, k are mapped by SiLU then unit L2 norm per token on load */
    LA_FUSE_OUT_RMSNORM = 2,   /* each output row is RMS-normalised and weighted */
    LA_FUSE_OUT_LAYERNORM = 4  /* each output row is layer-normalised, weighted and shifted */
} la_fuse;

typedef enum la_vla_readout {
    LA_VLA_RATIO = 0,   /* the page's output: ELU+1 on keys and queries, o = S phi(q) / (n . phi(q)) */
    LA_VLA_LINEAR = 1   /* o = S q, the key only normalised */
} la_vla_readout;

typedef enum la_variant {
    LA_RETENTION = 0,   /* la_chunk_fwd */
    LA_GLA = 1,         /* gla_chunk_fwd */
    LA_GDELTA = 2,      /* gdelta_chunk_fwd */
    LA_MAMBA2 = 3,      /* mamba2_chunk_fwd */
    LA_GDELTA_FUSED = 4 /* gdelta_chunk_fwd_fused with LA_FUSE_QK_SILU_L2 */
} la_variant;

/*
 * Workspace needed by a chunk entry point of `variant` for these sizes, in
 * bytes, written to *bytes (0 when none is needed).  Checks the sizes like the
 * entry point does (status and la_last_error() as there); the pointers of the
 * entry point are not involved.  For bf16 storage, retention and the scalar
 * data-dependent decay run in a single pass with no workspace when
 * B * H * (d_v / 16) >= 128 (the memory stays on chip), and so does GLA at
 * chunk 64 with d_k of 64 or 128 under the same rule (one sequence's log-gate
 * rows, padded to whole chunks, below 2^31 bytes); on the other shapes the
 * memory entering every chunk goes from a state pass to an output pass:
 * B * H * ceil(T / chunk) * d_v * d_k * 2 bytes.  For the gated
 * delta rule in bf16, with N = B * H * ceil(T / chunk) and a(x) = x rounded up
 * to a multiple of 256: at chunk 64 with d_k >= 32, the factor T_U of every
 * chunk (chunk x chunk bf16) and its cumulative log-gates (chunk float32),
 * a(N*chunk*chunk*2) + a(N*chunk*4) bytes, plus the mapped keys and queries,
 * 2 a(N*chunk*d_k*2), for gdelta_chunk_fwd_fused with LA_FUSE_QK_SILU_L2
 * (query with LA_GDELTA_FUSED); at chunks 16 and 32 or d_k = 16, the WY factor
 * W (chunk x d_k bf16), the pseudo-values (d_v x chunk float32), the
 * cumulative log-gates and the memory entering the chunk (d_v x d_k bf16),
 * a(N*chunk*d_k*2) + a(N*d_v*chunk*4) + a(N*chunk*4) + a(N*d_v*d_k*2) bytes,
 * plus the mapped keys a(N*chunk*d_k*2) with LA_GDELTA_FUSED.  fp32 storage
 * needs none.
 */
la_status la_chunk_workspace_size(la_variant variant, int B, int H, int T, int dk, int dv,
                                  int chunk, la_dtype dtype, size_t* bytes);

/*
 * Retention with a fixed decay per head (RetNet; "Scrivere meglio nella
 * memoria", section "Dimenticare: i gate", scalar-decay equation with
 * alpha_t = gamma_h; the RetNet page, multi-scale retention):
 *     S_t = gamma_h S_{t-1} + v_t k_t^T,   o_t = S_t q_t.
 * log_gamma [H] float32 holds log(gamma_h) (<= 0 for a decay; 0 is pure
 * accumulation).
 */
la_status la_chunk_fwd(const void* q, const void* k, const void* v,
                       const float* log_gamma,
                       const float* s0, void* o, float* s_out,
                       int B, int H, int T, int dk, int dv, int chunk,
                       la_dtype dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * Scalar data-dependent decay, the Mamba-2 row of the transition table
 * ("Scrivere meglio nella memoria", section "Dimenticare: i gate", scalar-decay
 * equation with alpha_t produced from the input at every step):
 *     S_t = alpha_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t.
 * log_alpha [B][H][T] float32 holds log(alpha_t) (<= 0), one per token and
 * head.  Only the recurrence is covered, not the rest of a Mamba-2 layer.
 */
la_status mamba2_chunk_fwd(const void* q, const void* k, const void* v,
                           const float* log_alpha,
                           const float* s0, void* o, float* s_out,
                           int B, int H, int T, int dk, int dv, int chunk,
                           la_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Gated linear attention: a data-dependent gate per key channel ("Scrivere
 * meglio nella memoria", section "Dimenticare: i gate", diagonal-gate
 * equation):
 *     S_t = S_{t-1} Diag(alpha_t) + v_t k_t^T,   o_t = S_t q_t.
 * log_alpha [B][H][T][d_k] float32 holds log(alpha_t) (<= 0).  For bf16
 * storage the decays inside a chunk are factorised per 16-token tile (tokens
 * 16m .. 16m + 15 of the chunk): q and k are rescaled by e^(+-(G - m)) around
 * a reference m, the cumulative log-gate just before the tile, moved down to
 * 80 above the one at the tile's last token when the tile's gates sum below
 * -80.  So for every key channel the log-gates of each such tile must sum to
 * at least -160 (the factors stay within e^(+-80), inside the fp32 / bf16
 * range with room for |q|, |k| <= 100); beyond that the output is not
 * defined.  gla_chunk_bwd has the same bound.
 * fp32 storage evaluates every decay directly and has none.
 */
la_status gla_chunk_fwd(const void* q, const void* k, const void* v,
                        const float* log_alpha,
                        const float* s0, void* o, float* s_out,
                        int B, int H, int T, int dk, int dv, int chunk,
                        la_dtype dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Gated delta rule (Gated DeltaNet; "Scrivere meglio nella memoria", section
 * "Unire oblio e correzione: Gated DeltaNet"):
 *     S_t = S_{t-1} [alpha_t (I - beta_t k_t k_t^T)] + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * evaluated per chunk through the WY / pseudo-value representation (section
 * "Correggere: la delta rule": one triangular system per chunk, only the
 * end-of-chunk memory passed on).  log_alpha [B][H][T] float32 holds
 * log(alpha_t) (<= 0); beta [B][H][T] float32 the write strength (in [0, 1]
 * for a stable memory with unit-norm keys).
 */
la_status gdelta_chunk_fwd(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           const float* s0, void* o, float* s_out,
                           int B, int H, int T, int dk, int dv, int chunk,
                           la_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * gdelta_chunk_fwd with DeltaNet's feature map and output norm fused in
 * ("Scrivere meglio nella memoria": the SiLU followed by L2 normalisation that
 * DeltaNet puts on the projections producing k and q, introduction section
 * "Superiore"; the RMS norm on the output that stabilises its readout).  `fuse`
 * is a bitwise OR of la_fuse flags:
 *  - LA_FUSE_QK_SILU_L2: q and k hold the projections before the map; every
 *    token's q and k become silu(x) / ||silu(x)||_2 (a zero row stays zero), in
 *    fp32, stored as bf16 before they enter the products (fp32 storage: kept
 *    in fp32);
 *  - LA_FUSE_OUT_RMSNORM: every output row o (d_v values) becomes
 *    o / sqrt(mean(o^2) + o_norm_eps) * o_norm_weight, with o_norm_weight
 *    [d_v] float32 (required with this flag) and o_norm_eps >= 0.
 * s_out is the memory itself, not affected by the output norm.  fuse == 0 is
 * gdelta_chunk_fwd.  With LA_FUSE_QK_SILU_L2 and bf16 storage the workspace
 * also holds the mapped keys: its size comes from la_chunk_workspace_size with
 * LA_GDELTA_FUSED.  Other arguments and errors as for gdelta_chunk_fwd; an
 * unknown flag is LA_ERR_INVALID.
 */
la_status gdelta_chunk_fwd_fused(const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta,
                                 const float* s0, void* o, float* s_out,
                                 const float* o_norm_weight, float o_norm_eps, int fuse,
                                 int B, int H, int T, int dk, int dv, int chunk,
                                 la_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * gdelta_chunk_fwd for callers that cannot allocate device memory (code under
 * stream capture, serving loops and harnesses that forbid hipMalloc): no
 * workspace argument.  The workspace is instead a fixed array of
 * LA_NOALLOC_SCRATCH_BYTES bytes in the library's own device memory, one copy
 * per device, held until the process ends.  A shape whose workspace
 * (la_chunk_workspace_size with LA_GDELTA) is larger is LA_ERR_UNSUPPORTED and
 * nothing is enqueued.  Every call on a device uses that device's one array
 * and leaves its last contents there: calls whose work overlaps in time on one
 * device (different streams or host threads) race and give undefined results;
 * calls on one stream are ordered and safe.  The first call on a device looks
 * the array's address up (with that device current); no call allocates.
 * Other arguments, behaviour and errors as for gdelta_chunk_fwd.
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
la_status gdelta_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta,
                                   const float* s0, void* o, float* s_out,
                                   int B, int H, int T, int dk, int dv, int chunk,
                                   la_dtype dtype, void* stream);

/*
 * gla_chunk_fwd with GLA's output norm fused in (the gates page, section
 * "Correggere: la delta rule", names a LayerNorm as GLA's output norm, beside
 * DeltaNet's RMS norm).  With fuse = LA_FUSE_OUT_LAYERNORM every output row o
 * (d_v values of one token and head) becomes
 *     (o - mean(o)) / sqrt(var(o) + o_norm_eps) * o_norm_weight + o_norm_bias,
 * var the mean squared deviation over the d_v values, in fp32, before o is
 * stored; o_norm_weight [d_v] float32 is required, o_norm_bias [d_v] float32
 * may be NULL (no shift), o_norm_eps >= 0.  For bf16 storage the output pass
 * normalises each row while it holds it (no extra pass over o); fp32 storage
 * normalises the stored rows in one more pass.  s_out is the memory itself.
 * fuse == 0 is gla_chunk_fwd; any other flag is LA_ERR_INVALID.  Workspace,
 * other arguments, errors and the gate bound as for gla_chunk_fwd.
 */
la_status gla_chunk_fwd_fused(const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* s0, void* o, float* s_out,
                              const float* o_norm_weight, const float* o_norm_bias, float o_norm_eps,
                              int fuse, int B, int H, int T, int dk, int dv, int chunk,
                              la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * la_chunk_fwd and mamba2_chunk_fwd with an output norm (the gates page, section
 * "Correggere: la delta rule": an output normalisation after the readout, a
 * LayerNorm in GLA and an RMS norm in DeltaNet; here either one, chosen by fuse).
 * fuse = LA_FUSE_OUT_RMSNORM: every output row o (d_v values of one token and
 * head) becomes o / sqrt(mean(o^2) + o_norm_eps) * o_norm_weight, and
 * o_norm_bias must be NULL.  fuse = LA_FUSE_OUT_LAYERNORM: the row becomes
 * (o - mean(o)) / sqrt(var(o) + o_norm_eps) * o_norm_weight + o_norm_bias
 * (o_norm_bias may be NULL: no shift).  o_norm_weight, o_norm_bias [d_v]
 * float32; o_norm_eps >= 0; statistics in fp32.  The value channels of a row
 * are computed by several workgroups, so the norm is a pass over the stored
 * rows after the chunk kernels (bf16 rows in place, rounded once more).
 * Any other fuse value is LA_ERR_INVALID.  s_out is the memory itself.
 * Workspace, other arguments and errors as for la_chunk_fwd / mamba2_chunk_fwd.
 */
la_status la_chunk_fwd_fused(const void* q, const void* k, const void* v,
                             const float* log_gamma, const float* s0, void* o, float* s_out,
                             const float* o_norm_weight, const float* o_norm_bias,
                             float o_norm_eps, int fuse, int B, int H, int T, int dk, int dv,
                             int chunk, la_dtype dtype, void* workspace,
                             size_t workspace_bytes, void* stream);
la_status mamba2_chunk_fwd_fused(const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* s0, void* o,
                                 float* s_out, const float* o_norm_weight,
                                 const float* o_norm_bias, float o_norm_eps, int fuse,
                                 int B, int H, int T, int dk, int dv, int chunk,
                                 la_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * One decode token for N sequences x H heads with a per-key-channel gate (the
 * recurrent form of the RetNet page, section on retention: the same two
 * gestures for every token at constant memory; a fixed decay is the constant
 * gate):
 *     S <- S Diag(alpha);  S <- S + v k^T;  o = S q.
 * q, k [N][H][d_k], v and o [N][H][d_v] in `dtype`; alpha [N][H][d_k] float32;
 * s [N][H][d_v][d_k] float32 is read and overwritten in place.
 * N == 0 or H == 0 is a no-op.  No chunk argument: `chunk` rules do not apply.
 */
la_status la_recurrent_step(const void* q, const void* k, const void* v,
                            const float* alpha, float* s, void* o,
                            int N, int H, int dk, int dv,
                            la_dtype dtype, void* stream);

/*
 * One decode token for N sequences x H heads under the gated delta rule
 * ("Scrivere meglio nella memoria", section "Unire oblio e correzione: Gated
 * DeltaNet"; the recurrent form of the RetNet page):
 *     S <- S [alpha (I - beta k k^T)] + beta v k^T;  o = S q.
 * q, k [N][H][d_k], v and o [N][H][d_v] in `dtype`; alpha and beta [N][H]
 * float32 (one gate in (0, 1] and one write strength per sequence and head);
 * s [N][H][d_v][d_k] float32 is read and overwritten in place.  Errors as for
 * la_recurrent_step.
 */
la_status gdelta_recurrent_step(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, float* s, void* o,
                                int N, int H, int dk, int dv,
                                la_dtype dtype, void* stream);

/*
 * Backward of la_chunk_fwd (retention) and mamba2_chunk_fwd (scalar
 * data-dependent decay): reverse-mode gradients of the recurrence ("Scrivere
 * meglio nella memoria", section "Dimenticare: i gate", scalar decay) through
 * the chunkwise form of the RetNet page.  Given dout [B][H][T][d_v] (the
 * gradient of the loss with respect to o, in `dtype`) and, optionally, ds_out
 * [B][H][d_v][d_k] float32 (with respect to the final memory; NULL = zero),
 * writes dq, dk [B][H][T][d_k] and dv [B][H][T][d_v] in `dtype`, the gate
 * gradient (la_chunk_bwd: dlog_gamma [H], summed over the batch and the
 * tokens of each head; mamba2_chunk_bwd: dlog_alpha [B][H][T]) and, if ds0 is
 * not NULL, ds0 [B][H][d_v][d_k] float32 (with respect to s0).  The forward
 * inputs (q, k, v, the gate, s0) are those of the forward call; the forward
 * is not needed beforehand (its carry is recomputed).  Only LA_BF16 storage
 * (LA_ERR_UNSUPPORTED otherwise).  The workspace size comes from
 * la_chunk_bwd_workspace_size: with N = B * H * ceil(T / chunk) and a(x) = x
 * rounded up to a multiple of 256, 2 a(N*d_v*d_k*2) + a(B*H*d_v*d_k*4) +
 * a(B*H*T*4) bytes.  Other conventions and errors as for the forward.
 */
la_status la_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk,
                                      la_dtype dtype, size_t* bytes);
la_status la_chunk_bwd(const void* q, const void* k, const void* v, const float* log_gamma,
                       const float* s0, const void* dout, const float* ds_out,
                       void* dq, void* dk_, void* dv_, float* dlog_gamma, float* ds0,
                       int B, int H, int T, int dk, int dv, int chunk,
                       la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);
la_status mamba2_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* s0, const void* dout, const float* ds_out,
                           void* dq, void* dk_, void* dv_, float* dlog_alpha, float* ds0,
                           int B, int H, int T, int dk, int dv, int chunk,
                           la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Variational linear attention over whole sequences ("Riepilogo Tecnico:
 * Attenzione Lineare Variazionale (VLA)", sections 2.1-2.3), token by token
 * in one launch.  Per (b, h) and token t, with the inverse penalty A (d_k x d_k)
 * beside the memory S:
 *     z = A u_t;  A <- A - z z^T / (1 + u_t . z)        (M <- M + u_t u_t^T)
 *     a = A k^ / |A k^|
 *     S <- S + (v_t - S k^) a^T
 * and the readout after the write, chosen by `readout`:
 *  - LA_VLA_RATIO (section 2.3, last paragraph: a ratio of recurrences as in
 *    standard linear attention, with the ELU+1 feature map phi(x) = x + 1 for
 *    x > 0, e^x otherwise, on keys and queries): k^ = phi(k_t) / |phi(k_t)|,
 *    the denominator vector n [d_k] follows the same write with the value 1,
 *    n <- n + (1 - n . k^) a, and o_t = S phi(q_t) / (n . phi(q_t));
 *  - LA_VLA_LINEAR: k^ = k_t / |k_t| and o_t = S q_t (no map, no normaliser).
 * q, k, u [B][H][T][d_k] and v, o [B][H][T][d_v] in `dtype` (u_t is the penalty
 * direction added at token t); A starts at a0 [B][H][d_k][d_k] float32 or,
 * when a0 is NULL, at I / lambda0 (lambda0 > 0 and finite); S at s0
 * [B][H][d_v][d_k] float32 or zeros; n (ratio readout) at n0 [B][H][d_k]
 * float32 or zeros.  s_out, a_out and n_out (float32, optional) receive the
 * final S, A and n; each may equal its starting pointer.  n0 and n_out are
 * not used by the linear readout.  Arithmetic is fp32 throughout.  A zero key
 * (linear) or a zero denominator (ratio) gives Inf or NaN, which propagates.
 * B, H or T == 0 is valid (outputs the starting state or its default).  d_k,
 * d_v in {16, 32, 64, 128} (LA_ERR_UNSUPPORTED otherwise); an unknown readout
 * is LA_ERR_INVALID.  Pointers 16-byte aligned; no workspace.  Errors as for
 * la_chunk_fwd.
 */
la_status vla_fwd(const void* q, const void* k, const void* v, const void* u,
                  float lambda0, const float* a0, const float* s0, const float* n0,
                  void* o, float* s_out, float* a_out, float* n_out, int readout,
                  int B, int H, int T, int dk, int dv, la_dtype dtype, void* stream);

/*
 * One VLA decode token for N sequences x H heads: vla_fwd with T = 1 and the
 * memory s [N][H][d_v][d_k], the inverse penalty a [N][H][d_k][d_k] and, for
 * the ratio readout, the denominator vector n [N][H][d_k] (float32; required
 * with LA_VLA_RATIO, unused with LA_VLA_LINEAR) read and overwritten in place.
 * q, k, u [N][H][d_k], v and o [N][H][d_v] in `dtype`.  N == 0 or H == 0 is a
 * no-op.  Errors as for la_recurrent_step.
 */
la_status vla_recurrent_step(const void* q, const void* k, const void* v, const void* u,
                             float* s, float* a, float* n, void* o, int readout,
                             int N, int H, int dk, int dv, la_dtype dtype, void* stream);

/*
 * Backward of gla_chunk_fwd (gate per key channel): reverse-mode gradients of
 * the diagonal-gate recurrence ("Scrivere meglio nella memoria", section
 * "Dimenticare: i gate") through the chunkwise form, with the forward's
 * per-16-token factorisation of the decays.  As la_chunk_bwd, with the gate
 * log_alpha [B][H][T][d_k] float32 and its gradient dlog_alpha [B][H][T][d_k]
 * float32.  The workspace size comes from gla_chunk_bwd_workspace_size: with
 * N and a(x) as for la_chunk_bwd, 2 a(N*d_v*d_k*2) + a(B*H*d_v*d_k*4) bytes.
 * Only LA_BF16 storage.
 */
la_status gla_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk,
                                       la_dtype dtype, size_t* bytes);
la_status gla_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* s0, const void* dout, const float* ds_out,
                        void* dq, void* dk_, void* dv_, float* dlog_alpha, float* ds0,
                        int B, int H, int T, int dk, int dv, int chunk,
                        la_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of gdelta_chunk_fwd: reverse-mode gradients of the gated delta rule
 * ("Scrivere meglio nella memoria", section "Unire oblio e correzione: Gated
 * DeltaNet") for L = <dout, o> + <ds_out, s_out>, through the chunkwise UT form
 * (section "Correggere: la delta rule").  The memory entering every chunk is
 * recomputed chunk by chunk (at chunk 64 with d_k >= 32: by the forward single
 * pass, which also records the chunk's pseudo-values), the memory's gradient is
 * carried back through the chunks the same way (at chunk 64: the single pass
 * run in reverse), and every chunk's input gradients then follow independently.
 * Inputs as for gdelta_chunk_fwd plus dout [B][H][T][d_v] (bf16) and ds_out
 * [B][H][d_v][d_k] float32 (NULL: zero); outputs dq, dk [B][H][T][d_k] and dv
 * [B][H][T][d_v] (bf16), dlog_alpha and dbeta [B][H][T] float32, and, if not
 * NULL, ds0 [B][H][d_v][d_k] float32.  The forward is not needed beforehand.
 * Only LA_BF16 storage; chunk 16, 32 or 64.  The workspace size comes from
 * gdelta_chunk_bwd_workspace_size: with N = B * H * ceil(T / chunk), C = chunk
 * and a(x) as for la_chunk_bwd: 2 a(N*C*C*2) + a(N*C*4) (T_U, T, the gates),
 * a(N*d_k*C*2) + 2 a(N*d_k*d_k*2) (each chunk's linear map, chunks 16 and 32),
 * 3 a(N*d_v*d_k*2) (its write, the memory entering it and the gradient leaving
 * it), 3 a(N*C*d_v*2) (the pseudo-values U and R and dU, chunk 64) and a
 * scratch of a(min(N, 512) * (6 C d_k + 3 C d_v + 6 C^2 + d_k^2) * 4) bytes.
 * Other conventions and errors as for la_chunk_bwd.
 */
la_status gdelta_chunk_bwd_workspace_size(int B, int H, int T, int dk, int dv, int chunk,
                                          la_dtype dtype, size_t* bytes);
la_status gdelta_chunk_bwd(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* s0, const void* dout, const float* ds_out,
                           void* dq, void* dk_, void* dv_, float* dlog_alpha, float* dbeta, float* ds0,
                           int B, int H, int T, int dk, int dv, int chunk, la_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* la_status_str(la_status status);

/* Message describing the last non-OK status returned to the calling thread
 * (thread-local; empty if none).  Valid until the next call on that thread. */
const char* la_last_error(void);

/* ABI version: (major << 16) | minor (2.0: workspace arguments; 2.1:
 * mamba2_chunk_fwd; 2.2: gdelta_recurrent_step; 2.3: gdelta_chunk_fwd_fused;
 * 2.4: la_chunk_bwd, mamba2_chunk_bwd; 2.5: vla_fwd, vla_recurrent_step; 2.6: gla_chunk_bwd;
 * 2.7: single-pass retention and scalar-decay forward, no workspace at B * H * d_v / 16 >= 128;
 * 3.0: vla_fwd and vla_recurrent_step take the readout and the denominator vector;
 * 3.1: gdelta_chunk_fwd_noalloc; 3.2: gla_chunk_fwd_fused; 3.3: gdelta_chunk_bwd;
 * 3.4: la_chunk_fwd_fused, mamba2_chunk_fwd_fused). */
int la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLR_H */
