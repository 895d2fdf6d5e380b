"""GPU parity of variational linear attention (vla_fwd, vla_recurrent_step) against the
fp64 oracle, through the C ABI, on seeded inputs (VLA summary page, "Riepilogo Tecnico:
Attenzione Lineare Variazionale (VLA)", section 2.3), for both readouts: the page's ratio
of recurrences with the ELU+1 feature map, and o = S q.

Bounds: o within the stated bf16 (max |d| <= 2e-2, and <= 1e-2 of max |o|) and fp32
(<= 1e-4) tolerances; the memory S, the inverse penalty A and the denominator vector n,
fp32 in both storage types (the arithmetic is fp32 throughout), within 1e-3 of their
largest entry."""

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


def _st(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _rel(x, ref):
    return np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-30)


def _check(label, dtype, o, o_ref, S, S_ref, A, A_ref, n=None, n_ref=None):
    err = np.max(np.abs(o - o_ref)) if o.size else 0.0
    scale = max(np.max(np.abs(o_ref)) if o_ref.size else 0.0, 1e-30)
    serr, aerr = _rel(S, S_ref), _rel(A, A_ref)
    nerr = _rel(n, n_ref) if n_ref is not None else 0.0
    msg = f"{label} max|do|={err:.3e} max|o|={scale:.3e} rel dS={serr:.3e} rel dA={aerr:.3e} rel dn={nerr:.3e}"
    print(msg, flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S)) and np.all(np.isfinite(A)), msg
    if dtype == "f32":
        assert err <= 1e-4, msg
    else:
        assert err <= 2e-2 and err <= 1e-2 * scale, msg
    assert serr <= 1e-3 and aerr <= 1e-3 and nerr <= 1e-3, msg


# (B, H, T, d_k, d_v): block tails (16-token staging), every head size, one token, none
SHAPES = [(1, 2, 37, 16, 16), (2, 1, 100, 32, 64), (1, 2, 130, 64, 32), (2, 2, 200, 128, 128),
          (1, 1, 1, 128, 128), (1, 3, 16, 128, 16), (2, 1, 24, 16, 128), (1, 2, 0, 64, 64)]


@pytest.mark.parametrize("readout", ["ratio", "linear"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("state", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_vla_parity(shape, state, dtype, readout):
    B, H, T, dk, dv = shape
    w = synthetic.vla_inputs(B, H, T, dk, dv, dtype=dtype, seed=700 + sum(shape), with_state=state, lambda0=0.8,
                             readout=readout)
    st = _st(dtype)
    print(f"vla_fwd {shape} state={state} {dtype} {readout}", flush=True)
    o, S, A, n = api.vla_fwd(_t(w.q, st), _t(w.k, st), _t(w.v, st), _t(w.u, st), lambda0=w.lambda0, a0=_t(w.a0),
                             s0=_t(w.s0), n0=_t(w.n0), readout=readout)
    torch.cuda.synchronize()
    o_ref, S_ref, A_ref, n_ref = orc.vla_recurrent(w.q, w.k, w.v, w.u, lambda0=w.lambda0, s0=w.s0, a0=w.a0,
                                                   n0=w.n0, readout=readout)
    assert (n is None) == (readout == "linear")
    _check(f"vla {shape} state={state} {dtype} {readout}", dtype, o.float().cpu().numpy(), o_ref, S.cpu().numpy(),
           S_ref, A.cpu().numpy(), A_ref, None if n is None else n.cpu().numpy(), n_ref)


@pytest.mark.parametrize("readout", ["ratio", "linear"])
def test_vla_in_place_continuation(readout):
    """s_out, a_out and n_out may alias s0, a0 and n0: two calls in place equal one call."""
    B, H, T, dk, dv = 2, 2, 90, 64, 64
    w = synthetic.vla_inputs(B, H, T, dk, dv, dtype="bf16", seed=7, with_state=True, readout=readout)
    q, k, v, u = (_t(x, torch.bfloat16) for x in (w.q, w.k, w.v, w.u))
    S, A, N = _t(w.s0), _t(w.a0), _t(w.n0)
    outs = []
    for sl in (slice(0, 41), slice(41, T)):
        o, _, _, _ = api.vla_fwd(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(), v[:, :, sl].contiguous(),
                                 u[:, :, sl].contiguous(), a0=A, s0=S, n0=N, s_out=S, a_out=A, n_out=N,
                                 readout=readout)
        outs.append(o)
    torch.cuda.synchronize()
    o_ref, S_ref, A_ref, n_ref = orc.vla_recurrent(w.q, w.k, w.v, w.u, s0=w.s0, a0=w.a0, n0=w.n0, readout=readout)
    _check(f"vla in place {readout}", "bf16", torch.cat(outs, dim=2).float().cpu().numpy(), o_ref, S.cpu().numpy(),
           S_ref, A.cpu().numpy(), A_ref, N.cpu().numpy() if readout == "ratio" else None, n_ref)


@pytest.mark.parametrize("readout", ["ratio", "linear"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dims", [(128, 128), (64, 32), (16, 16)])
def test_vla_decode_steps(dims, dtype, readout):
    """Five decode tokens in place on the memory, the inverse penalty and the denominator."""
    dk, dv = dims
    N, H, steps = 6, 3, 5
    w = synthetic.vla_decode_inputs(N, H, dk, dv, steps=steps, dtype=dtype, seed=dk + dv, readout=readout)
    st = _st(dtype)
    s, a, n = _t(w.s0), _t(w.a0), _t(w.n0)
    s_ref, a_ref = w.s0.astype(np.float64), w.a0.astype(np.float64)
    n_ref = w.n0.astype(np.float64) if readout == "ratio" else None
    for i in range(steps):
        o = api.vla_recurrent_step(_t(w.q[i], st), _t(w.k[i], st), _t(w.v[i], st), _t(w.u[i], st), s, a, n=n,
                                   readout=readout)
        torch.cuda.synchronize()
        o_ref, s_ref, a_ref, n_ref = orc.vla_decode_step(w.q[i], w.k[i], w.v[i], w.u[i], s_ref, a_ref, n_ref,
                                                         readout=readout)
        _check(f"vla decode {dims} {dtype} {readout} step {i}", dtype, o.float().cpu().numpy(), o_ref,
               s.cpu().numpy(), s_ref, a.cpu().numpy(), a_ref, n.cpu().numpy() if readout == "ratio" else None,
               n_ref)


def test_vla_full_size_sampled():
    """The B8 H16 T4096 d128 workload (ratio readout) in the launch configuration the bench
    times; the oracle follows two sampled (sequence, head) pairs over all 4096 tokens."""
    name = "vla_b8h16_t4096_d128"
    w = synthetic.config_inputs(name)
    o, S, A, n = api.vla_fwd(_t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16),
                             _t(w.u, torch.bfloat16), lambda0=w.lambda0)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (7, 13)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, S_ref, A_ref, n_ref = orc.vla_recurrent(w.q[sl], w.k[sl], w.v[sl], w.u[sl], lambda0=w.lambda0)
        _check(f"{name} (b={b}, h={h})", "bf16", o[sl].float().cpu().numpy(), o_ref, S[sl].cpu().numpy(), S_ref,
               A[sl].cpu().numpy(), A_ref, n[sl].cpu().numpy(), n_ref)
