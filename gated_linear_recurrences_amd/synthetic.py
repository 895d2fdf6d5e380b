"""Seeded synthetic inputs for the recurrences (shared by the tests and the benchmark).

This module only draws random numbers and rounds them to the storage type. It
holds none of the recurrences' arithmetic: no decay, no write, no readout. The
same arrays feed the HIP path (uploaded as-is) and the fp64 oracle (upcast
exactly), so a parity test measures the kernels' arithmetic, not input
quantisation.

Recipes (numpy ``default_rng(seed)``; draws happen in the order listed):

* ``retention`` - q, k, v iid N(0, 1) * scale, rounded to the storage type; a
  per-head log-decay ``log(1 - 2^(-5-h))`` (multi-scale retention, one decay per
  head, h = 0..H-1) or a given constant decay.
* ``gla`` - q, k, v as above, then one log-gate per (b, h, t, key channel):
  ``logsigmoid(x) / 16`` with x ~ N(0, 1) (the log of a sigmoid gate raised to
  1/16, the GLA temperature), fp32.
* ``gdelta`` - q and k are ``L2-normalise(SiLU(x))`` of x ~ N(0, 1), rounded to
  the storage type; v ~ N(0, 1); then one write strength
  ``beta = sigmoid(x)`` and one log-decay ``-softplus(x) / 8`` per (b, h, t), fp32.
* ``decode`` - the state ``S ~ N(0, 0.01)`` (variance 0.01, i.e. std 0.1) fp32,
  then per step q, k, v ~ N(0, 1) / sqrt(d) and a per-key-channel gate
  ``sigmoid(N(2, 1))`` in (0, 1), fp32.

bf16 values are produced by rounding fp32 to nearest-even, the rounding the
device's own conversion uses; they are returned in float32 containers holding
exactly representable bf16 values.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "round_to_bf16",
    "Workload",
    "retention_inputs",
    "gla_inputs",
    "gdelta_inputs",
    "decode_inputs",
    "vla_inputs",
    "vla_decode_inputs",
    "CONFIGS",
    "config_inputs",
]


def round_to_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); float32 container."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = (u + bias) & np.uint32(0xFFFF0000)
    return out.view(np.float32)


def _store(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _logsigmoid(x):
    return -np.logaddexp(0.0, -x)


def _softplus(x):
    return np.logaddexp(0.0, x)


@dataclass
class Workload:
    """One seeded input set. Arrays are numpy, float32 containers (bf16-exact when
    ``dtype == 'bf16'``); the gates are always float32."""

    kind: str                  # 'retention' | 'mamba2' | 'gla' | 'gdelta' | 'decode'
    dtype: str                 # storage type of q, k, v, o: 'bf16' | 'f32'
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    chunk: int = 0
    log_gamma: Optional[np.ndarray] = None   # retention [H]
    log_alpha: Optional[np.ndarray] = None   # gla [B,H,T,dk]; mamba2, gdelta [B,H,T]
    beta: Optional[np.ndarray] = None        # gdelta [B,H,T]
    alpha: Optional[np.ndarray] = None       # decode [N,H,dk] (or [steps,N,H,dk]); delta decode [steps,N,H]
    s0: Optional[np.ndarray] = None          # [B,H,dv,dk] fp32
    u: Optional[np.ndarray] = None           # vla penalty directions [B,H,T,dk] (decode: [steps,N,H,dk])
    a0: Optional[np.ndarray] = None          # vla inverse penalty [B,H,dk,dk] fp32
    n0: Optional[np.ndarray] = None          # vla readout denominator vector [B,H,dk] fp32
    lambda0: float = 1.0                     # vla: A_0 = I / lambda0 when a0 is None
    meta: dict = field(default_factory=dict)


def retention_inputs(B, H, T, dk, dv, *, chunk=64, dtype="bf16", seed=0, scale=None,
                     gamma=None, with_state=False):
    """q, k, v ~ N(0,1)*scale; per-head decay 1 - 2^(-5-h) unless a constant ``gamma``."""
    rng = np.random.default_rng(seed)
    scale = (1.0 / np.sqrt(dk)) if scale is None else scale
    q = _store(rng.standard_normal((B, H, T, dk)) * scale, dtype)
    k = _store(rng.standard_normal((B, H, T, dk)) * scale, dtype)
    v = _store(rng.standard_normal((B, H, T, dv)) * scale, dtype)
    if gamma is None:
        g = 1.0 - np.power(2.0, -5.0 - np.arange(H, dtype=np.float64))
    else:
        g = np.full(H, float(gamma))
    log_gamma = np.log(g).astype(np.float32)
    s0 = (rng.standard_normal((B, H, dv, dk)).astype(np.float32) * np.float32(0.1)
          if with_state else None)
    return Workload("retention", dtype, q, k, v, chunk=chunk, log_gamma=log_gamma, s0=s0)


def mamba2_inputs(B, H, T, dk, dv, *, chunk=64, dtype="bf16", seed=0, scale=None,
                  temperature=16.0, with_state=False):
    """q, k, v ~ N(0,1)*scale; one log-gate logsigmoid(N(0,1)) / temperature per token and head
    (the per-channel recipe of the GLA workload, drawn once per token)."""
    rng = np.random.default_rng(seed)
    scale = (1.0 / np.sqrt(dk)) if scale is None else scale
    q = _store(rng.standard_normal((B, H, T, dk)) * scale, dtype)
    k = _store(rng.standard_normal((B, H, T, dk)) * scale, dtype)
    v = _store(rng.standard_normal((B, H, T, dv)) * scale, dtype)
    log_alpha = (_logsigmoid(rng.standard_normal((B, H, T))) / temperature).astype(np.float32)
    s0 = (rng.standard_normal((B, H, dv, dk)).astype(np.float32) * np.float32(0.1)
          if with_state else None)
    return Workload("mamba2", dtype, q, k, v, chunk=chunk, log_alpha=log_alpha, s0=s0)


def gla_inputs(B, H, T, dk, dv, *, chunk=64, dtype="bf16", seed=0, scale=None,
               temperature=16.0, with_state=False):
    """q, k, v ~ N(0,1)*scale; log-gate logsigmoid(N(0,1)) / temperature per key channel."""
    rng = np.random.default_rng(seed)
    scale = (1.0 / np.sqrt(dk)) if scale is None else scale
    q = _store(rng.standard_normal((B, H, T, dk)) * scale, dtype)
    k = _store(rng.standard_normal((B, H, T, dk)) * scale, dtype)
    v = _store(rng.standard_normal((B, H, T, dv)) * scale, dtype)
    log_alpha = (_logsigmoid(rng.standard_normal((B, H, T, dk))) / temperature).astype(np.float32)
    s0 = (rng.standard_normal((B, H, dv, dk)).astype(np.float32) * np.float32(0.1)
          if with_state else None)
    return Workload("gla", dtype, q, k, v, chunk=chunk, log_alpha=log_alpha, s0=s0)


def _silu_l2(x):
    y = x * _sigmoid(x)
    return y / np.linalg.norm(y, axis=-1, keepdims=True)


def gdelta_inputs(B, H, T, dk, dv, *, chunk=64, dtype="bf16", seed=0, with_state=False, raw_qk=False):
    """q, k = L2(SiLU(N(0,1))); v ~ N(0,1); beta = sigmoid(N(0,1)); log alpha = -softplus(N(0,1))/8.
    With ``raw_qk`` q and k are the N(0,1) draws themselves (the projections before the feature
    map, for the fused entry point), rounded to the storage type."""
    rng = np.random.default_rng(seed)
    fmap = (lambda x: x) if raw_qk else _silu_l2
    q = _store(fmap(rng.standard_normal((B, H, T, dk))), dtype)
    k = _store(fmap(rng.standard_normal((B, H, T, dk))), dtype)
    v = _store(rng.standard_normal((B, H, T, dv)), dtype)
    beta = _sigmoid(rng.standard_normal((B, H, T))).astype(np.float32)
    log_alpha = (-_softplus(rng.standard_normal((B, H, T))) / 8.0).astype(np.float32)
    s0 = (rng.standard_normal((B, H, dv, dk)).astype(np.float32) * np.float32(0.1)
          if with_state else None)
    return Workload("gdelta", dtype, q, k, v, chunk=chunk, log_alpha=log_alpha, beta=beta, s0=s0)


def decode_inputs(N, H, dk, dv, *, steps=1, dtype="bf16", seed=0):
    """Initial state S ~ N(0, 0.01) fp32, then ``steps`` fresh tokens: q, k, v ~ N(0,1)/sqrt(dk)
    and a gate sigmoid(N(2,1)) per key channel. Token arrays carry a leading step axis."""
    rng = np.random.default_rng(seed)
    s0 = (rng.standard_normal((N, H, dv, dk)) * 0.1).astype(np.float32)
    scale = 1.0 / np.sqrt(dk)
    q = np.empty((steps, N, H, dk), np.float32)
    k = np.empty((steps, N, H, dk), np.float32)
    v = np.empty((steps, N, H, dv), np.float32)
    a = np.empty((steps, N, H, dk), np.float32)
    for s in range(steps):
        q[s] = _store(rng.standard_normal((N, H, dk)) * scale, dtype)
        k[s] = _store(rng.standard_normal((N, H, dk)) * scale, dtype)
        v[s] = _store(rng.standard_normal((N, H, dv)) * scale, dtype)
        a[s] = _sigmoid(rng.standard_normal((N, H, dk)) + 2.0).astype(np.float32)
    return Workload("decode", dtype, q, k, v, alpha=a, s0=s0)


def gdelta_decode_inputs(N, H, dk, dv, *, steps=1, dtype="bf16", seed=0):
    """Gated-delta decode: initial state S ~ N(0, 0.01) fp32, then ``steps`` fresh tokens with
    the gated-delta workload's recipe: q, k = L2(SiLU(N(0,1))), v ~ N(0,1), beta = sigmoid(N(0,1))
    and alpha = exp(-softplus(N(0,1)) / 8) per sequence and head. Leading step axis."""
    rng = np.random.default_rng(seed)
    s0 = (rng.standard_normal((N, H, dv, dk)) * 0.1).astype(np.float32)
    q = np.empty((steps, N, H, dk), np.float32)
    k = np.empty((steps, N, H, dk), np.float32)
    v = np.empty((steps, N, H, dv), np.float32)
    a = np.empty((steps, N, H), np.float32)
    b = np.empty((steps, N, H), np.float32)
    for s in range(steps):
        q[s] = _store(_silu_l2(rng.standard_normal((N, H, dk))), dtype)
        k[s] = _store(_silu_l2(rng.standard_normal((N, H, dk))), dtype)
        v[s] = _store(rng.standard_normal((N, H, dv)), dtype)
        b[s] = _sigmoid(rng.standard_normal((N, H))).astype(np.float32)
        a[s] = np.exp(-_softplus(rng.standard_normal((N, H))) / 8.0).astype(np.float32)
    return Workload("gdelta_decode", dtype, q, k, v, alpha=a, beta=b, s0=s0)


def _penalty_inverse(lead, dk, lambda0, rng):
    """A symmetric positive-definite starting inverse penalty: I / lambda0 plus a symmetric
    perturbation of spectral norm below 0.1 / lambda0."""
    G = rng.standard_normal(lead + (dk, dk))
    P = (G + np.swapaxes(G, -1, -2)) / (2.0 * np.sqrt(dk))
    return ((np.eye(dk) + 0.04 * P) / lambda0).astype(np.float32)


def vla_inputs(B, H, T, dk, dv, *, dtype="bf16", seed=0, with_state=False, lambda0=1.0, readout="ratio"):
    """Variational linear attention: v ~ N(0,1), u ~ N(0,1)/sqrt(dk) (the penalty direction
    added per token); q, k ~ N(0,1) for the ratio readout (unit scale: its ELU+1 feature map
    sees both of its branches) or N(0,1)/sqrt(dk) for the linear one (o = S q at the scale of
    the other workloads); A_0 = I / lambda0 (with_state: a perturbed SPD A_0, S_0 ~ N(0, 0.01)
    and a positive denominator vector n_0 ~ U(0.8, 1.6)/sqrt(dk), the scale it settles at)."""
    rng = np.random.default_rng(seed)
    sc = 1.0 if readout == "ratio" else 1.0 / np.sqrt(dk)
    q = _store(rng.standard_normal((B, H, T, dk)) * sc, dtype)
    k = _store(rng.standard_normal((B, H, T, dk)) * sc, dtype)
    v = _store(rng.standard_normal((B, H, T, dv)), dtype)
    u = _store(rng.standard_normal((B, H, T, dk)) / np.sqrt(dk), dtype)
    s0 = a0 = n0 = None
    if with_state:
        s0 = (rng.standard_normal((B, H, dv, dk)) * 0.1).astype(np.float32)
        a0 = _penalty_inverse((B, H), dk, lambda0, rng)
        n0 = (rng.uniform(0.8, 1.6, (B, H, dk)) / np.sqrt(dk)).astype(np.float32)
    return Workload("vla", dtype, q, k, v, s0=s0, u=u, a0=a0, n0=n0, lambda0=lambda0)


def vla_decode_inputs(N, H, dk, dv, *, steps=1, dtype="bf16", seed=0, lambda0=1.0, readout="ratio"):
    """VLA decode: S_0 ~ N(0, 0.01) fp32, a perturbed SPD A_0, n_0 ~ U(0.8, 1.6)/sqrt(dk),
    then ``steps`` fresh tokens with the sequence workload's recipe for that readout. Leading
    step axis on q, k, v, u."""
    rng = np.random.default_rng(seed)
    s0 = (rng.standard_normal((N, H, dv, dk)) * 0.1).astype(np.float32)
    a0 = _penalty_inverse((N, H), dk, lambda0, rng)
    n0 = (rng.uniform(0.8, 1.6, (N, H, dk)) / np.sqrt(dk)).astype(np.float32)
    sc = 1.0 if readout == "ratio" else 1.0 / np.sqrt(dk)
    q = _store(rng.standard_normal((steps, N, H, dk)) * sc, dtype)
    k = _store(rng.standard_normal((steps, N, H, dk)) * sc, dtype)
    v = _store(rng.standard_normal((steps, N, H, dv)), dtype)
    u = _store(rng.standard_normal((steps, N, H, dk)) / np.sqrt(dk), dtype)
    return Workload("vla_decode", dtype, q, k, v, s0=s0, u=u, a0=a0, n0=n0, lambda0=lambda0)


# The five workloads the throughput and parity figures are quoted on, and the scalar
# data-dependent decay at the GLA workload's shape.
CONFIGS = {
    "retention_t64_d16_f32": dict(kind="retention", B=1, H=1, T=64, dk=16, dv=16, chunk=16,
                                  dtype="f32", gamma=0.9, scale=1.0, seed=1),
    "retention_b4h8_t2048_d128": dict(kind="retention", B=4, H=8, T=2048, dk=128, dv=128,
                                      chunk=64, dtype="bf16", seed=2),
    "gla_b8h16_t4096_d128": dict(kind="gla", B=8, H=16, T=4096, dk=128, dv=128, chunk=64,
                                 dtype="bf16", seed=3),
    "gdelta_b4h16_t8192_d128": dict(kind="gdelta", B=4, H=16, T=8192, dk=128, dv=128, chunk=64,
                                    dtype="bf16", seed=4),
    "decode_n512h32_d128": dict(kind="decode", N=512, H=32, dk=128, dv=128, steps=1000,
                                dtype="bf16", seed=5),
    "mamba2_b8h16_t4096_d128": dict(kind="mamba2", B=8, H=16, T=4096, dk=128, dv=128, chunk=64,
                                    dtype="bf16", seed=6),
    "vla_b8h16_t4096_d128": dict(kind="vla", B=8, H=16, T=4096, dk=128, dv=128, chunk=0, dtype="bf16",
                                 seed=8),
}


def config_inputs(name, *, steps=None, T=None):
    """Inputs of one named workload; ``T`` (chunk forms) or ``steps`` (decode) may be reduced."""
    c = dict(CONFIGS[name])
    kind = c.pop("kind")
    seed = c.pop("seed")
    if kind == "decode":
        return decode_inputs(c["N"], c["H"], c["dk"], c["dv"],
                             steps=c["steps"] if steps is None else steps,
                             dtype=c["dtype"], seed=seed)
    Tn = c["T"] if T is None else T
    if kind == "retention":
        return retention_inputs(c["B"], c["H"], Tn, c["dk"], c["dv"], chunk=c["chunk"],
                                dtype=c["dtype"], seed=seed, scale=c.get("scale"),
                                gamma=c.get("gamma"))
    if kind == "gla":
        return gla_inputs(c["B"], c["H"], Tn, c["dk"], c["dv"], chunk=c["chunk"],
                          dtype=c["dtype"], seed=seed)
    if kind == "mamba2":
        return mamba2_inputs(c["B"], c["H"], Tn, c["dk"], c["dv"], chunk=c["chunk"],
                             dtype=c["dtype"], seed=seed)
    if kind == "vla":
        return vla_inputs(c["B"], c["H"], Tn, c["dk"], c["dv"], dtype=c["dtype"], seed=seed)
    if kind == "gdelta":
        return gdelta_inputs(c["B"], c["H"], Tn, c["dk"], c["dv"], chunk=c["chunk"],
                             dtype=c["dtype"], seed=seed)
    raise ValueError(kind)
