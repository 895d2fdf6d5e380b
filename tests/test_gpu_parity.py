"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element.

Gates (written here, applied to every comparison):
  * float32 storage: max |o - o_ref| <= 1e-4 and the same for the final memory;
  * bfloat16 storage (bf16 MFMA operands, fp32 accumulation and memory):
    max |o - o_ref| <= 2e-2, and - because outputs can be small - also
    max |o - o_ref| / max |o_ref| <= 1e-2 and max |S - S_ref| / max |S_ref| <= 1e-2;
  * decode (fp32 memory, one step is a handful of fp32 FMAs per element):
    max |o - o_ref| <= 2e-2 and, relative to max |o_ref|, <= 1e-2 for bf16 outputs (their
    own rounding is 2^-9 relative) and <= 1e-4 for fp32 outputs; memory relative <= 1e-5.
The oracle reads exactly the values uploaded to the GPU (bf16 values upcast), so the
comparison measures the kernels' arithmetic.
"""

import numpy as np
import pytest
import torch

import oracle as orc
from gated_linear_recurrences_amd import api, synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _t(x, dtype=torch.float32):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def _storage(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def run_gpu(w, s0=None, chunk=None, o=None, s_out=None):
    """Run a chunk workload through the binding; returns (o, S_T) as float64 numpy."""
    st = _storage(w)
    q, k, v = _t(w.q, st), _t(w.k, st), _t(w.v, st)
    s0_t = _t(s0 if s0 is not None else w.s0)
    c = chunk or w.chunk
    if w.kind == "retention":
        out, S = api.la_chunk_fwd(q, k, v, _t(w.log_gamma), chunk=c, s0=s0_t, o=o, s_out=s_out)
    elif w.kind == "mamba2":
        out, S = api.mamba2_chunk_fwd(q, k, v, _t(w.log_alpha), chunk=c, s0=s0_t, o=o, s_out=s_out)
    elif w.kind == "gla":
        out, S = api.gla_chunk_fwd(q, k, v, _t(w.log_alpha), chunk=c, s0=s0_t, o=o, s_out=s_out)
    else:
        out, S = api.gdelta_chunk_fwd(q, k, v, _t(w.log_alpha), _t(w.beta), chunk=c, s0=s0_t, o=o,
                                      s_out=s_out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64)


def run_oracle(w, s0=None, chunk=None):
    s0 = s0 if s0 is not None else w.s0
    c = chunk or w.chunk
    if w.kind == "retention":
        return orc.retention_chunkwise(w.q, w.k, w.v, w.log_gamma, c, s0=s0)
    if w.kind == "mamba2":
        return orc.scalar_chunkwise(w.q, w.k, w.v, w.log_alpha, c, s0=s0)
    if w.kind == "gla":
        return orc.gla_chunkwise(w.q, w.k, w.v, w.log_alpha, c, s0=s0)
    return orc.gdelta_chunkwise(w.q, w.k, w.v, w.log_alpha, w.beta, c, s0=s0)


def assert_parity(w, o, S, o_ref, S_ref, label="", normed=False):
    """``normed``: o is RMS-normalised per row. The norm divides each row by its RMS, so an
    error of the recurrence's output grows by 1/RMS in absolute terms; the absolute 2e-2
    bound of the recurrence's output does not carry over, the relative one does (and the
    recurrence's own output is checked under both with the norm off)."""
    err = np.max(np.abs(o - o_ref)) if o.size else 0.0
    scale = max(np.max(np.abs(o_ref)) if o_ref.size else 0.0, 1e-30)
    serr = np.max(np.abs(S - S_ref))
    sscale = max(np.max(np.abs(S_ref)), 1e-30)
    msg = f"{label} max|do|={err:.3e} max|o|={scale:.3e} max|dS|={serr:.3e} max|S|={sscale:.3e}"
    print(msg)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S)), msg
    if w.dtype == "f32":
        assert err <= 1e-4, msg
        assert serr <= 1e-4 * max(1.0, sscale), msg
    else:
        assert normed or err <= 2e-2, msg
        assert err / scale <= 1e-2, msg
        assert serr / sscale <= 1e-2, msg


def make(kind, B, H, T, dk, dv, chunk, dtype, seed, state):
    if kind == "retention":
        return synthetic.retention_inputs(B, H, T, dk, dv, chunk=chunk, dtype=dtype, seed=seed, with_state=state)
    if kind == "mamba2":
        return synthetic.mamba2_inputs(B, H, T, dk, dv, chunk=chunk, dtype=dtype, seed=seed, with_state=state)
    if kind == "gla":
        return synthetic.gla_inputs(B, H, T, dk, dv, chunk=chunk, dtype=dtype, seed=seed, with_state=state)
    return synthetic.gdelta_inputs(B, H, T, dk, dv, chunk=chunk, dtype=dtype, seed=seed, with_state=state)


KINDS = ["retention", "mamba2", "gla", "gdelta"]

# (B, H, T, d_k, d_v, chunk): several chunks, ragged tails, every supported head size and chunk
SMALL_SHAPES = [
    (1, 2, 100, 16, 16, 16),
    (2, 1, 77, 32, 64, 32),
    (1, 2, 130, 64, 32, 64),
    (2, 2, 200, 128, 128, 64),
    (1, 1, 64, 128, 16, 16),
    (1, 1, 1, 64, 64, 64),
]


# ----------------------------------------------------------------------------- float32 path

@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("state", [False, True])
def test_f32_chunk_parity(kind, shape, state):
    w = make(kind, *shape, dtype="f32", seed=100 + sum(shape), state=state)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    assert_parity(w, o, S, o_ref, S_ref, f"{kind} f32 {shape} state={state}")


def test_retention_t64_d16_f32_config():
    """The fp32 retention workload: T=64, d=16, gamma=0.9, q/k/v iid N(0,1), chunk 16."""
    w = synthetic.config_inputs("retention_t64_d16_f32")
    o, S = run_gpu(w)
    o_ref, S_ref = orc.retention_recurrent(w.q, w.k, w.v, w.log_gamma)
    assert_parity(w, o, S, o_ref, S_ref, "retention_t64_d16_f32")


# ----------------------------------------------------------------------------- bfloat16 path

@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("state", [False, True])
def test_bf16_chunk_parity(kind, shape, state):
    w = make(kind, *shape, dtype="bf16", seed=200 + sum(shape), state=state)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    assert_parity(w, o, S, o_ref, S_ref, f"{kind} bf16 {shape} state={state}")


# (B, H, T, d_k, d_v, chunk) with B * H * d_v / 16 >= 128: retention and the scalar decay take
# the single-pass forward there (no workspace). Every d_k, d_v and chunk, value slices of 16,
# 32 and 64 channels (at chunk 64 with 256 or more slices of 64: two value tiles per chain
# wave), ragged tails, a lone partial chunk, T = 1 and T = 0.
SINGLE_PASS_SHAPES = [
    (2, 8, 100, 16, 128, 16),     # 16-channel slices, d_k = 16
    (4, 8, 77, 32, 64, 32),
    (8, 8, 130, 64, 32, 64),
    (16, 16, 45, 128, 16, 64),    # one partial chunk, d_v = 16
    (4, 16, 200, 128, 128, 64),   # 32-channel slices
    (16, 16, 40, 32, 128, 16),    # 32-channel slices, chunk 16
    (2, 64, 1, 64, 64, 64),
    (8, 8, 0, 64, 32, 64),
    (4, 8, 150, 16, 64, 64),      # chunk 64 (q taken from registers), d_k = 16: half the lanes idle
    (4, 8, 99, 32, 128, 64),      # chunk 64, d_k = 32
    (4, 64, 130, 128, 128, 64),   # 64-channel slices, two value tiles per chain wave
    (16, 16, 70, 64, 64, 64),     # one 64-channel slice per sequence, d_k = 64
    (32, 8, 1, 32, 64, 64),       # 64-channel slices, T = 1
]


@pytest.mark.parametrize("kind", ["retention", "mamba2"])
@pytest.mark.parametrize("shape", SINGLE_PASS_SHAPES)
@pytest.mark.parametrize("state", [False, True])
def test_bf16_single_pass_parity(kind, shape, state):
    B, H, T, dk, dv, chunk = shape
    assert B * H * dv // 16 >= 128
    assert api.workspace_size(kind, *shape) == 0
    w = make(kind, *shape, dtype="bf16", seed=500 + sum(shape), state=state)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    if T == 0:
        np.testing.assert_array_equal(S, w.s0.astype(np.float64) if state else 0.0)
        return
    assert_parity(w, o, S, o_ref, S_ref, f"{kind} single pass {shape} state={state}")


@pytest.mark.parametrize("shape", [(2, 64, 70, 16, 128, 64), (4, 64, 70, 16, 128, 64)])
def test_bf16_gla_dk16_many_heads(shape):
    """GLA's state pass with d_k = 16 (one wave per workgroup) and enough heads that each
    wave takes 4, then 8, value tiles of 16 channels: the configurations whose group of
    chunks per barrier is limited by the register ring rather than by LDS."""
    w = make("gla", *shape, dtype="bf16", seed=700 + sum(shape), state=True)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    assert_parity(w, o, S, o_ref, S_ref, f"gla d_k=16 {shape}")


# GLA takes its own single pass at chunk 64 with d_k of 64 or 128 under the same rule: the
# chunk-64 shapes above (16-, 32- and 64-channel value slices, ragged tails, a lone partial
# chunk, T = 1 and T = 0).
GLA_SINGLE_PASS_SHAPES = [s for s in SINGLE_PASS_SHAPES if s[5] == 64 and s[3] >= 64]


@pytest.mark.parametrize("shape", GLA_SINGLE_PASS_SHAPES)
@pytest.mark.parametrize("state", [False, True])
def test_bf16_gla_single_pass_parity(shape, state):
    B, H, T, dk, dv, chunk = shape
    assert api.workspace_size("gla", *shape) == 0
    w = make("gla", *shape, dtype="bf16", seed=600 + sum(shape), state=state)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    if T == 0:
        np.testing.assert_array_equal(S, w.s0.astype(np.float64) if state else 0.0)
        return
    assert_parity(w, o, S, o_ref, S_ref, f"gla single pass {shape} state={state}")


@pytest.mark.parametrize("kind", ["retention", "mamba2"])
@pytest.mark.parametrize("shape", [(4, 8, 150, 128, 64, 64), (2, 64, 70, 64, 32, 32)])
def test_bf16_single_pass_strong_decay(kind, shape):
    """Gates far from 1: log alpha in [-4, -2] per token (a chunk's gates then sum below
    2^-100, where the scalar gate's e^(G_i) e^(-G_j) product form would overflow, so the
    kernel takes e^(G_i - G_j) per element) and log gamma = -2.5 per head. Outputs are
    dominated by the last few tokens; compared like every bf16 case."""
    B, H, T, dk, dv, chunk = shape
    assert B * H * dv // 16 >= 128
    w = make(kind, *shape, dtype="bf16", seed=900 + sum(shape), state=True)
    rng = np.random.default_rng(901)
    if kind == "retention":
        w.log_gamma = np.full((H,), -2.5, dtype=np.float32)
    else:
        w.log_alpha = rng.uniform(-4.0, -2.0, size=(B, H, T)).astype(np.float32)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    assert_parity(w, o, S, o_ref, S_ref, f"{kind} strong decay {shape}")


@pytest.mark.parametrize("name", ["retention_b4h8_t2048_d128", "gla_b8h16_t4096_d128",
                                  "gdelta_b4h16_t8192_d128", "mamba2_b8h16_t4096_d128"])
def test_bf16_full_config_parity(name):
    """Full-size workloads in the launch configuration the benchmark times, every output."""
    w = synthetic.config_inputs(name)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    assert_parity(w, o, S, o_ref, S_ref, name)


# ----------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
def test_empty_sequence_hands_state_through(kind, dtype):
    w = make(kind, 2, 2, 0, 64, 32, 64, dtype, 7, True)
    o, S = run_gpu(w)
    assert o.shape == (2, 2, 0, 32)
    np.testing.assert_array_equal(S, w.s0.astype(np.float64))
    w.s0 = None
    _, S = run_gpu(w)
    np.testing.assert_array_equal(S, 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("heads", [(1, 2), (4, 8)])
def test_resume_and_in_place_state(kind, dtype, heads):
    """Two calls (first 93 tokens, then the rest from s_out, in place s0 == s_out) match one
    call. (4, 8) heads at d_v = 64 take the single-pass forward for retention and the scalar
    decay, (1, 2) the two-pass one."""
    B, H = heads
    w = make(kind, B, H, 160, 128, 64, 64, dtype, 8, True)
    o_full, S_full = run_gpu(w)
    st = _storage(w)

    def part(sl, s):
        sub = make(kind, B, H, 160, 128, 64, 64, dtype, 8, True)
        sub.q, sub.k, sub.v = w.q[..., sl, :], w.k[..., sl, :], w.v[..., sl, :]
        if kind == "gla":
            sub.log_alpha = w.log_alpha[..., sl, :]
        elif kind == "mamba2":
            sub.log_alpha = w.log_alpha[..., sl]
        elif kind == "gdelta":
            sub.log_alpha, sub.beta = w.log_alpha[..., sl], w.beta[..., sl]
        q, k, v = _t(sub.q, st), _t(sub.k, st), _t(sub.v, st)
        if kind == "retention":
            out, _ = api.la_chunk_fwd(q, k, v, _t(w.log_gamma), chunk=64, s0=s, s_out=s)
        elif kind == "gla":
            out, _ = api.gla_chunk_fwd(q, k, v, _t(sub.log_alpha), chunk=64, s0=s, s_out=s)
        elif kind == "mamba2":
            out, _ = api.mamba2_chunk_fwd(q, k, v, _t(sub.log_alpha), chunk=64, s0=s, s_out=s)
        else:
            out, _ = api.gdelta_chunk_fwd(q, k, v, _t(sub.log_alpha), _t(sub.beta), chunk=64, s0=s, s_out=s)
        return out

    s = _t(w.s0)
    o1 = part(slice(0, 93), s)
    o2 = part(slice(93, 160), s)
    torch.cuda.synchronize()
    o = torch.cat([o1, o2], dim=-2).float().cpu().numpy()
    o_ref, S_ref = run_oracle(w)
    assert_parity(w, o.astype(np.float64), s.cpu().numpy().astype(np.float64), o_ref, S_ref, f"resume {kind}")
    if dtype == "f32":
        np.testing.assert_allclose(o, o_full, atol=2e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("heads", [(2, 2), (4, 4)])
def test_deterministic(kind, dtype, heads):
    """No atomics on the path: two runs give bit-identical outputs ((4, 4) heads at d_v = 128:
    the single-pass forward for retention and the scalar decay)."""
    w = make(kind, *heads, 150, 128, 128, 64, dtype, 9, True)
    o1, S1 = run_gpu(w)
    o2, S2 = run_gpu(w)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


# ----------------------------------------------------------------------------- fused feature map / output norm

def _fused_reference(w, weight, eps, qk, norm):
    """The oracle around the fused entry point, all in fp64: SiLU + L2 on the raw q, k (kept
    in fp64: the kernel's own rounding of the mapped rows is part of the error measured),
    the gated-delta chunkwise form, then the RMS norm of each output row."""
    q, k = w.q, w.k
    if qk:
        q, k = orc.silu_l2(q), orc.silu_l2(k)
    o, S = orc.gdelta_chunkwise(q, k, w.v, w.log_alpha, w.beta, w.chunk, s0=w.s0)
    if norm:
        o = orc.rms_norm(o, weight, eps)
    return o, S


FUSED_SHAPES = [(1, 2, 100, 16, 16, 16), (2, 1, 77, 32, 64, 32), (2, 2, 200, 128, 128, 64), (1, 1, 64, 128, 16, 16),
                (1, 2, 130, 64, 32, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flags", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("shape", FUSED_SHAPES)
def test_gdelta_fused_parity(shape, flags, dtype):
    qk, norm = flags
    B, H, T, dk, dv, c = shape
    w = synthetic.gdelta_inputs(B, H, T, dk, dv, chunk=c, dtype=dtype, seed=500 + sum(shape), with_state=True,
                                raw_qk=qk)
    weight = np.random.default_rng(sum(shape)).uniform(0.5, 1.5, dv).astype(np.float32)
    st = _storage(w)
    out, S = api.gdelta_chunk_fwd_fused(_t(w.q, st), _t(w.k, st), _t(w.v, st), _t(w.log_alpha), _t(w.beta),
                                        chunk=c, qk_silu_l2=qk, o_norm_weight=_t(weight) if norm else None,
                                        o_norm_eps=1e-6, s0=_t(w.s0))
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    o_ref, S_ref = _fused_reference(w, weight, 1e-6, qk, norm)
    assert_parity(w, o, S.cpu().numpy().astype(np.float64), o_ref, S_ref, f"fused {flags} {dtype} {shape}",
                  normed=norm)


def test_gdelta_fused_full_size_parity():
    """The gated-delta workload's shape (B4 H16 T8192, d 128) from raw q, k with the RMS norm."""
    w = synthetic.gdelta_inputs(4, 16, 8192, 128, 128, chunk=64, dtype="bf16", seed=4, raw_qk=True)
    weight = np.random.default_rng(4).uniform(0.5, 1.5, 128).astype(np.float32)
    out, S = api.gdelta_chunk_fwd_fused(_t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16),
                                        _t(w.log_alpha), _t(w.beta), chunk=64, o_norm_weight=_t(weight))
    torch.cuda.synchronize()
    o_ref, S_ref = _fused_reference(w, weight, 1e-6, True, True)
    assert_parity(w, out.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64), o_ref, S_ref,
                  "fused full size", normed=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("shape", FUSED_SHAPES)
def test_gla_layernorm_fused_parity(shape, bias, dtype):
    """GLA with its output LayerNorm fused in against the oracle's layer_norm of the GLA
    chunkwise output (fp64), under the same gates as the plain forward (relative bound for
    the normalised rows); the memory is untouched by the norm."""
    B, H, T, dk, dv, c = shape
    w = synthetic.gla_inputs(B, H, T, dk, dv, chunk=c, dtype=dtype, seed=700 + sum(shape), with_state=True)
    rng = np.random.default_rng(sum(shape) + 1)
    weight = rng.uniform(0.5, 1.5, dv).astype(np.float32)
    b = rng.standard_normal(dv).astype(np.float32) * 0.5 if bias else None
    st = _storage(w)
    out, S = api.gla_chunk_fwd_fused(_t(w.q, st), _t(w.k, st), _t(w.v, st), _t(w.log_alpha), _t(weight),
                                     o_norm_bias=_t(b) if bias else None, o_norm_eps=1e-5, chunk=c, s0=_t(w.s0))
    torch.cuda.synchronize()
    o_gla, S_ref = orc.gla_chunkwise(w.q, w.k, w.v, w.log_alpha, c, s0=w.s0)
    o_ref = orc.layer_norm(o_gla, weight, b, 1e-5)
    assert_parity(w, out.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64), o_ref, S_ref,
                  f"gla layernorm bias={bias} {dtype} {shape}", normed=True)


def test_gla_layernorm_fused_full_size_parity():
    """The GLA workload's shape (B8 H16 T4096, d 128) with the LayerNorm fused in: the
    oracle's chunkwise output on 8 of the 128 sequences (one per batch entry, head h = b),
    then layer_norm."""
    w = synthetic.config_inputs("gla_b8h16_t4096_d128")
    rng = np.random.default_rng(3)
    weight = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    b = rng.standard_normal(128).astype(np.float32) * 0.5
    out, S = api.gla_chunk_fwd_fused(_t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16),
                                     _t(w.log_alpha), _t(weight), o_norm_bias=_t(b), o_norm_eps=1e-5, chunk=64)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    S = S.cpu().numpy().astype(np.float64)
    for bi in range(8):
        sl = (slice(bi, bi + 1), slice(bi, bi + 1))
        o_gla, S_ref = orc.gla_chunkwise(w.q[sl], w.k[sl], w.v[sl], w.log_alpha[sl], 64)
        assert_parity(w, o[sl], S[sl], orc.layer_norm(o_gla, weight, b, 1e-5), S_ref,
                      f"gla layernorm full size sequence {bi}", normed=True)


# (B, H, T, d_k, d_v, chunk): two-pass shapes (few sequences), single-pass ones (chunk 64 on the
# gated delta rule's pass, 16-, 32- and 64-channel slices; chunk 16 on fused_kernel)
NORM_SHAPES = [(1, 2, 100, 16, 16, 16), (2, 1, 77, 32, 64, 32), (4, 8, 150, 128, 64, 64), (4, 16, 130, 128, 128, 64),
               (4, 64, 70, 128, 128, 64), (8, 8, 70, 64, 32, 16)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", ["rms", "layer", "layer_bias"])
@pytest.mark.parametrize("kind", ["retention", "mamba2"])
@pytest.mark.parametrize("shape", NORM_SHAPES)
def test_norm_fused_parity(shape, kind, norm, dtype):
    """Retention and the scalar decay with their output norm fused in, against the oracle's
    chunkwise output then rms_norm or layer_norm (fp64), under the relative bound of
    normalised rows; the memory is untouched by the norm."""
    B, H, T, dk, dv, c = shape
    w = make(kind, B, H, T, dk, dv, c, dtype, 800 + sum(shape), True)
    rng = np.random.default_rng(sum(shape) + 3)
    weight = rng.uniform(0.5, 1.5, dv).astype(np.float32)
    bias = rng.standard_normal(dv).astype(np.float32) * 0.5 if norm == "layer_bias" else None
    st = _storage(w)
    q, k, v = _t(w.q, st), _t(w.k, st), _t(w.v, st)
    kw = dict(o_norm_bias=_t(bias) if bias is not None else None, o_norm_eps=1e-5,
              norm="rms" if norm == "rms" else "layer", chunk=c, s0=_t(w.s0))
    if kind == "retention":
        out, S = api.la_chunk_fwd_fused(q, k, v, _t(w.log_gamma), _t(weight), **kw)
    else:
        out, S = api.mamba2_chunk_fwd_fused(q, k, v, _t(w.log_alpha), _t(weight), **kw)
    torch.cuda.synchronize()
    o_plain, S_ref = run_oracle(w)
    o_ref = orc.rms_norm(o_plain, weight, 1e-5) if norm == "rms" else orc.layer_norm(o_plain, weight, bias, 1e-5)
    assert_parity(w, out.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64), o_ref, S_ref,
                  f"{kind} {norm} {dtype} {shape}", normed=True)


# ----------------------------------------------------------------------------- backward

BWD_SHAPES = [(1, 2, 100, 16, 16, 16), (2, 1, 77, 32, 64, 32), (1, 2, 130, 64, 32, 64), (2, 2, 200, 128, 128, 64),
              (1, 1, 64, 128, 16, 16), (1, 1, 1, 64, 64, 64), (1, 2, 0, 64, 64, 64), (4, 8, 192, 128, 128, 64)]


def _bwd_gate(name, got, ref, floor=0.0):
    """Gradients are held to the forward's relative bound, max |d| <= 1e-2 max |ref|. A gate
    gradient is a sum over tokens of q.dq - k.dk terms that cancel (for retention over a
    whole head: a value near 1 from terms summing to 2e3 in absolute value), so it is held to
    1e-2 of its L2 norm plus ``floor``: 1e-3 of the norm of the same sums taken over the
    absolute values of the terms, i.e. each term's own error carried through the sum."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if floor:
        err, scale = np.linalg.norm(got - ref), np.linalg.norm(ref)
    else:
        err, scale = np.max(np.abs(got - ref)), np.max(np.abs(ref))
    bound = 1e-2 * max(scale, 1e-30) + floor
    msg = f"{name}: err={err:.3e} scale={scale:.3e} bound={bound:.3e}"
    print(msg)
    assert np.all(np.isfinite(got)), msg
    assert err <= bound, msg


def _gate_terms_floor(kind, q, k, dq, dk):
    """1e-3 of the L2 norm of the gate gradient's terms in absolute value: per token
    sum_{s >= t} |q_s.dq_s| + |k_s.dk_s| (scalar gates), per head the sum over the batch and
    the tokens of (s + 1) times the same (fixed gates); 4e-3 of the norm of the per-channel
    sums sum_{s >= t} |q_s[c] dq_s[c]| + |k_s[c] dk_s[c]| (GLA)."""
    if kind == "gla":
        # per-channel terms: no sum over d_k channels averages the rounding of dq[c] and
        # dk[c] (bf16 MFMA operands, relative 2^-8), so the floor is 4e-3 of the terms
        ab = np.abs(np.float64(q) * dq) + np.abs(np.float64(k) * dk)
        return 4e-3 * float(np.linalg.norm(np.flip(np.cumsum(np.flip(ab, 2), 2), 2)))
    ab = np.abs(np.einsum("bhtc,bhtc->bht", np.float64(q), dq)) + np.abs(np.einsum("bhtc,bhtc->bht", np.float64(k), dk))
    if kind == "retention":
        sc = (ab * (np.arange(ab.shape[-1]) + 1)).sum(axis=(0, 2))
    else:
        sc = np.flip(np.cumsum(np.flip(ab, -1), -1), -1)
    return 1e-3 * float(np.linalg.norm(sc))


@pytest.mark.parametrize("kind", ["retention", "mamba2", "gla"])
@pytest.mark.parametrize("shape", BWD_SHAPES)
@pytest.mark.parametrize("extras", [False, True])
def test_backward_parity(kind, shape, extras):
    """dq, dk, dv, the gate gradient and ds0 of the bf16 backward against the oracle's
    reverse-mode gradients of the recurrence, for L = <dout, o> (+ <ds_out, S_T>)."""
    B, H, T, dk, dv, c = shape
    w = make(kind, B, H, T, dk, dv, c, "bf16", 600 + sum(shape), extras)
    rng = np.random.default_rng(sum(shape))
    dout = synthetic.round_to_bf16(rng.standard_normal((B, H, T, dv)) / np.sqrt(dv)).astype(np.float32)
    ds_out = (rng.standard_normal((B, H, dv, dk)) * 0.1).astype(np.float32) if extras else None
    q, k, v = _t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16)
    if kind == "retention":
        dq, dk_, dv_, dg, ds0 = api.la_chunk_bwd(q, k, v, _t(w.log_gamma), _t(dout, torch.bfloat16), s0=_t(w.s0),
                                                 ds_out=_t(ds_out), chunk=c)
        ref = orc.retention_backward(w.q, w.k, w.v, w.log_gamma, dout, dS_T=ds_out, s0=w.s0)
    elif kind == "gla":
        dq, dk_, dv_, dg, ds0 = api.gla_chunk_bwd(q, k, v, _t(w.log_alpha), _t(dout, torch.bfloat16),
                                                  s0=_t(w.s0), ds_out=_t(ds_out), chunk=c)
        ref = orc.gla_backward(w.q, w.k, w.v, w.log_alpha, dout, dS_T=ds_out, s0=w.s0)
    else:
        dq, dk_, dv_, dg, ds0 = api.mamba2_chunk_bwd(q, k, v, _t(w.log_alpha), _t(dout, torch.bfloat16),
                                                     s0=_t(w.s0), ds_out=_t(ds_out), chunk=c)
        ref = orc.scalar_backward(w.q, w.k, w.v, w.log_alpha, dout, dS_T=ds_out, s0=w.s0)
    torch.cuda.synchronize()
    label = f"{kind} {shape} extras={extras}"
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk_, ref[1]), ("dv", dv_, ref[2]), ("ds0", ds0, ref[4])):
        if T == 0 and name != "ds0":
            continue
        _bwd_gate(f"{label} {name}", got.float().cpu().numpy(), r)
    floor = _gate_terms_floor(kind, w.q, w.k, ref[0], ref[1]) if T else 1e-30
    _bwd_gate(f"{label} dgate", dg.cpu().numpy(), ref[3], floor=floor)


def _gdelta_bwd(w, dout, ds_out, c, want_ds0=True):
    q, k, v = _t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16)
    out = api.gdelta_chunk_bwd(q, k, v, _t(w.log_alpha), _t(w.beta), _t(dout, torch.bfloat16), s0=_t(w.s0),
                               ds_out=_t(ds_out), chunk=c, want_ds0=want_ds0)
    torch.cuda.synchronize()
    return [None if x is None else x.float().cpu().numpy().astype(np.float64) for x in out]


def _gdelta_gate_grads_gate(label, got, ref):
    """d log alpha and dbeta are sums over the chunk's products that cancel: held to 2e-2 of
    their L2 norm (relative), the per-element gradients' 1e-2 doubled for the extra products
    (the triangular system's own gradient) that bf16 operands enter twice."""
    err, scale = np.linalg.norm(got - ref), np.linalg.norm(ref)
    msg = f"{label}: L2 err={err:.3e} L2 scale={scale:.3e}"
    print(msg)
    assert np.all(np.isfinite(got)), msg
    assert err <= 2e-2 * max(scale, 1e-30), msg


@pytest.mark.parametrize("shape", BWD_SHAPES)
@pytest.mark.parametrize("extras", [False, True])
def test_gdelta_backward_parity(shape, extras):
    """dq, dk, dv, d log alpha, dbeta and ds0 of gdelta_chunk_bwd against the oracle's reverse
    mode through the recurrent form, for L = <dout, o> (+ <ds_out, S_T>)."""
    B, H, T, dk, dv, c = shape
    w = synthetic.gdelta_inputs(B, H, T, dk, dv, chunk=c, dtype="bf16", seed=900 + sum(shape), with_state=extras)
    rng = np.random.default_rng(sum(shape) + 2)
    dout = synthetic.round_to_bf16(rng.standard_normal((B, H, T, dv)) / np.sqrt(dv)).astype(np.float32)
    ds_out = (rng.standard_normal((B, H, dv, dk)) * 0.1).astype(np.float32) if extras else None
    got = _gdelta_bwd(w, dout, ds_out, c)
    ref = orc.gdelta_backward(w.q, w.k, w.v, w.log_alpha, w.beta, dout, dS_T=ds_out, s0=w.s0)
    label = f"gdelta bwd {shape} extras={extras}"
    for name, gi, ri in (("dq", 0, 0), ("dk", 1, 1), ("dv", 2, 2), ("ds0", 5, 5)):
        if T == 0 and name != "ds0":
            continue
        _bwd_gate(f"{label} {name}", got[gi], ref[ri])
    if T:
        _gdelta_gate_grads_gate(f"{label} dlog_alpha", got[3], ref[3])
        _gdelta_gate_grads_gate(f"{label} dbeta", got[4], ref[4])


def test_gdelta_backward_full_size_parity():
    """The gated-delta workload's shape (B4 H16 T8192, d 128) through gdelta_chunk_bwd; one of the
    64 sequences checked against the oracle's reverse mode (every token)."""
    w = synthetic.config_inputs("gdelta_b4h16_t8192_d128")
    B, H, T, d = w.q.shape
    rng = np.random.default_rng(11)
    dout = synthetic.round_to_bf16(rng.standard_normal((B, H, T, d)) / np.sqrt(d)).astype(np.float32)
    got = _gdelta_bwd(w, dout, None, 64)
    b, h = 2, 5
    sl = (slice(b, b + 1), slice(h, h + 1))
    ref = orc.gdelta_backward(w.q[sl], w.k[sl], w.v[sl], w.log_alpha[sl], w.beta[sl], dout[sl])
    label = "gdelta bwd full size (b 2, h 5)"
    for name, gi in (("dq", 0), ("dk", 1), ("dv", 2), ("ds0", 5)):
        _bwd_gate(f"{label} {name}", got[gi][sl], ref[gi])
    _gdelta_gate_grads_gate(f"{label} dlog_alpha", got[3][sl], ref[3])
    _gdelta_gate_grads_gate(f"{label} dbeta", got[4][sl], ref[4])


@pytest.mark.parametrize("kind", ["mamba2", "gla"])
def test_backward_deterministic(kind):
    """No atomics: two backward calls give bit-identical gradients."""
    w = make(kind, 2, 2, 150, 128, 128, 64, "bf16", 9, True)
    q, k, v = _t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16)
    dout = torch.randn(w.v.shape, device=DEV).to(torch.bfloat16)
    fn = api.mamba2_chunk_bwd if kind == "mamba2" else api.gla_chunk_bwd
    r1 = fn(q, k, v, _t(w.log_alpha), dout, s0=_t(w.s0))
    r2 = fn(q, k, v, _t(w.log_alpha), dout, s0=_t(w.s0))
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


# ----------------------------------------------------------------------------- decode

def _decode_run(w, steps):
    st = _storage(w)
    s = _t(w.s0)
    outs = []
    for i in range(steps):
        o = api.la_recurrent_step(_t(w.q[i], st), _t(w.k[i], st), _t(w.v[i], st), _t(w.alpha[i]), s)
        outs.append(o.float())
    torch.cuda.synchronize()
    return [x.cpu().numpy().astype(np.float64) for x in outs], s.cpu().numpy().astype(np.float64)


def _decode_assert(o, o_ref, S, S_ref, label, dtype):
    err = np.max(np.abs(o - o_ref))
    scale = np.max(np.abs(o_ref))
    serr = np.max(np.abs(S - S_ref)) / np.max(np.abs(S_ref))
    msg = f"{label} max|do|={err:.3e} max|o|={scale:.3e} rel dS={serr:.3e}"
    print(msg)
    rel = 1e-2 if dtype == "bf16" else 1e-4
    assert err <= 2e-2 and err / scale <= rel and serr <= 1e-5, msg


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dims", [(3, 2, 16, 16), (2, 3, 32, 128), (4, 2, 128, 64), (2, 2, 64, 32)])
def test_decode_parity_small(dtype, dims):
    N, H, dk, dv = dims
    w = synthetic.decode_inputs(N, H, dk, dv, steps=5, dtype=dtype, seed=300 + dk + dv)
    outs, S = _decode_run(w, 5)
    S_ref = w.s0.astype(np.float64)
    for i in range(5):
        o_ref, S_ref = orc.decode_step(w.q[i], w.k[i], w.v[i], w.alpha[i], S_ref)
        _decode_assert(outs[i], o_ref, S if i == 4 else S_ref, S_ref, f"decode {dtype} {dims} step {i}", dtype)


def _gdelta_decode_run(w, steps):
    st = _storage(w)
    s = _t(w.s0)
    outs = []
    for i in range(steps):
        o = api.gdelta_recurrent_step(_t(w.q[i], st), _t(w.k[i], st), _t(w.v[i], st), _t(w.alpha[i]),
                                      _t(w.beta[i]), s)
        outs.append(o.float())
    torch.cuda.synchronize()
    return [x.cpu().numpy().astype(np.float64) for x in outs], s.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dims", [(3, 2, 16, 16), (2, 3, 32, 128), (4, 2, 128, 64), (2, 2, 64, 32), (2, 2, 128, 16)])
def test_gdelta_decode_parity_small(dtype, dims):
    N, H, dk, dv = dims
    w = synthetic.gdelta_decode_inputs(N, H, dk, dv, steps=5, dtype=dtype, seed=400 + dk + dv)
    outs, S = _gdelta_decode_run(w, 5)
    S_ref = w.s0.astype(np.float64)
    for i in range(5):
        o_ref, S_ref = orc.gdelta_decode_step(w.q[i], w.k[i], w.v[i], w.alpha[i], w.beta[i], S_ref)
        _decode_assert(outs[i], o_ref, S if i == 4 else S_ref, S_ref, f"gdelta decode {dtype} {dims} step {i}",
                       dtype)


def test_gdelta_decode_full_size_parity():
    """512 sequences x 32 heads, d = 128, three gated-delta steps, every output and the whole memory."""
    w = synthetic.gdelta_decode_inputs(512, 32, 128, 128, steps=3, dtype="bf16", seed=7)
    outs, S = _gdelta_decode_run(w, 3)
    S_ref = w.s0.astype(np.float64)
    for i in range(3):
        o_ref, S_ref = orc.gdelta_decode_step(w.q[i], w.k[i], w.v[i], w.alpha[i], w.beta[i], S_ref)
        _decode_assert(outs[i], o_ref, S if i == 2 else S_ref, S_ref, f"gdelta decode full step {i}", "bf16")


def test_decode_full_size_parity():
    """512 sequences x 32 heads, d = 128 (the decode workload's launch shape), three steps,
    every output and the whole memory."""
    w = synthetic.config_inputs("decode_n512h32_d128", steps=3)
    outs, S = _decode_run(w, 3)
    S_ref = w.s0.astype(np.float64)
    for i in range(3):
        o_ref, S_ref = orc.decode_step(w.q[i], w.k[i], w.v[i], w.alpha[i], S_ref)
        err = np.max(np.abs(outs[i] - o_ref))
        assert err <= 2e-2 and err / np.max(np.abs(o_ref)) <= 1e-2, (i, err)
    serr = np.max(np.abs(S - S_ref)) / np.max(np.abs(S_ref))
    assert serr <= 1e-5, serr


def test_decode_matches_recurrent_gla_over_many_steps():
    """Sixty decode steps on a handful of (sequence, head) pairs equal the oracle's recurrent
    GLA form over the same 60 tokens (the decode step is that recurrence, one token at a time)."""
    w = synthetic.decode_inputs(4, 2, 128, 128, steps=60, dtype="bf16", seed=31)
    outs, S = _decode_run(w, 60)
    seq = lambda x: np.moveaxis(x, 0, 2)          # [steps,N,H,d] -> [N,H,steps,d]
    o_ref, S_ref = orc.gla_recurrent(seq(w.q), seq(w.k), seq(w.v), np.log(seq(w.alpha)), s0=w.s0)
    o = np.stack(outs, axis=2)
    _decode_assert(o, o_ref, S, S_ref, "decode vs recurrent", "bf16")


# ----------------------------------------------------------------------------- launch shapes

# (B, H, T, d_k, d_v, chunk) chosen so that the two-pass forward's state pass takes each of
# its workgroup shapes (16 TV value channels per workgroup, TV = 1, 2, 4, 8, one or two waves
# per key tile, 1-4 chunks per barrier), with ragged tails and an initial memory
LAUNCH_SHAPES = [
    (4, 8, 130, 128, 128, 64),    # 32 sequences: TV = 2
    (8, 8, 97, 128, 128, 64),     # 64 sequences: TV = 4
    (8, 16, 70, 128, 128, 32),    # 128 sequences: TV = 8
    (2, 16, 150, 64, 64, 64),     # d = 64
    (16, 16, 40, 32, 128, 16),    # d_k = 32, chunk 16, 256 sequences
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", LAUNCH_SHAPES)
def test_bf16_launch_shapes(kind, shape):
    w = make(kind, *shape, dtype="bf16", seed=300 + sum(shape), state=True)
    o, S = run_gpu(w)
    o_ref, S_ref = run_oracle(w)
    assert_parity(w, o, S, o_ref, S_ref, f"{kind} bf16 {shape}")


# ----------------------------------------------------------------------------- workspace

def _ws_call(w, workspace):
    q, k, v = _t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16)
    if w.kind == "retention":
        out, S = api.la_chunk_fwd(q, k, v, _t(w.log_gamma), chunk=w.chunk, s0=_t(w.s0), workspace=workspace)
    else:
        out, S = api.gdelta_chunk_fwd(q, k, v, _t(w.log_alpha), _t(w.beta), chunk=w.chunk, s0=_t(w.s0),
                                      workspace=workspace)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), S.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kind", ["retention", "gdelta"])
def test_workspace_reused_and_garbage_filled(kind):
    """A caller's workspace may hold anything on entry and serve call after call."""
    w1 = make(kind, 2, 4, 300, 128, 128, 64, dtype="bf16", seed=41, state=True)
    w2 = make(kind, 2, 4, 200, 128, 128, 64, dtype="bf16", seed=42, state=True)
    need = api.workspace_size(kind, 2, 4, 300, 128, 128, 64)
    if kind == "retention":
        assert need == 2 * 4 * 5 * 128 * 128 * 2
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)   # NaN bit patterns
    for w in (w1, w2, w1):
        o, S = _ws_call(w, ws)
        o_ref, S_ref = run_oracle(w)
        assert_parity(w, o, S, o_ref, S_ref, f"{kind} workspace T={w.q.shape[2]}")


def test_workspace_too_small_is_rejected():
    w = make("gla", 1, 2, 100, 64, 64, 32, dtype="bf16", seed=43, state=False)
    need = api.workspace_size("gla", 1, 2, 100, 64, 64, 32)
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    q, k, v = _t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16)
    from gated_linear_recurrences_amd._native import GLRError
    with pytest.raises(GLRError, match="workspace too small"):
        api.gla_chunk_fwd(q, k, v, _t(w.log_alpha), chunk=32, workspace=ws)


# ----------------------------------------------------------------------------- HIP graphs

@pytest.mark.parametrize("kind,heads", [("retention", (4, 8)), ("retention", (1, 2)), ("mamba2", (4, 8)),
                                        ("gla", (2, 2)), ("gdelta", (2, 2))])
def test_graph_replay_matches_eager(kind, heads):
    """The forward entry points enqueue kernels only (no memset, no host synchronisation), so
    a caller may capture them in a HIP graph: every replay, with eager work and
    synchronisations between replays, equals the eager call bit for bit. (4, 8) heads take
    the single-pass forward for retention and the scalar decay, (1, 2) the two passes."""
    w = make(kind, *heads, 150, 128, 128, 64, "bf16", 61, True)
    st = _storage(w)
    q, k, v, s0 = _t(w.q, st), _t(w.k, st), _t(w.v, st), _t(w.s0)
    ws = torch.empty(max(api.workspace_size(kind, *heads, 150, 128, 128, 64), 16), dtype=torch.uint8, device=DEV)
    o = torch.empty(*heads, 150, 128, dtype=st, device=DEV)
    s_out = torch.empty(*heads, 128, 128, dtype=torch.float32, device=DEV)

    lg = _t(w.log_gamma) if kind == "retention" else None
    la = None if kind == "retention" else _t(w.log_alpha)
    be = _t(w.beta) if kind == "gdelta" else None

    def call():   # device buffers only: nothing is copied from the host during capture
        if kind == "retention":
            api.la_chunk_fwd(q, k, v, lg, chunk=64, s0=s0, o=o, s_out=s_out, workspace=ws)
        elif kind == "mamba2":
            api.mamba2_chunk_fwd(q, k, v, la, chunk=64, s0=s0, o=o, s_out=s_out, workspace=ws)
        elif kind == "gla":
            api.gla_chunk_fwd(q, k, v, la, chunk=64, s0=s0, o=o, s_out=s_out, workspace=ws)
        else:
            api.gdelta_chunk_fwd(q, k, v, la, be, chunk=64, s0=s0, o=o, s_out=s_out, workspace=ws)

    call()
    torch.cuda.synchronize()
    o_ref, s_ref = o.clone(), s_out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        o.zero_()
        s_out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s_out, s_ref), f"replay {rep}"
        call()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
