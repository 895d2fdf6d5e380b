"""Python binding of the C ABI with the same entry-point names.

Argument marshalling only: shape and dtype checks, output allocation through
PyTorch (device memory and streams are PyTorch's), and one call into
``libglr.so`` on the current HIP stream. Every step of the computation runs
in the library's kernels.
"""

import ctypes

import torch

from . import _native

__all__ = ["la_chunk_fwd", "mamba2_chunk_fwd", "gla_chunk_fwd", "gdelta_chunk_fwd", "gdelta_chunk_fwd_fused",
           "gdelta_chunk_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "gla_chunk_fwd_fused", "la_chunk_fwd_fused",
           "mamba2_chunk_fwd_fused",
           "la_chunk_bwd", "mamba2_chunk_bwd", "gla_chunk_bwd", "gdelta_chunk_bwd", "la_recurrent_step", "gdelta_recurrent_step",
           "vla_fwd", "vla_recurrent_step", "workspace_size", "bwd_workspace_size"]


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _native.LA_BF16
    if t.dtype == torch.float32:
        return _native.LA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(variant, dims, chunk, q, workspace):
    """The caller's workspace if given (checked by the library), else a fresh one
    from PyTorch's caching allocator of the size the library asks for."""
    B, H, T, dk, dv = dims
    need = _native.workspace_size(variant, B, H, T, dk, dv, chunk, _dtype_code(q))
    if workspace is not None:
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the device of q")
        return workspace, workspace.numel() * workspace.element_size()
    if need == 0:
        return None, 0
    return torch.empty(need, dtype=torch.uint8, device=q.device), need


def _chunk_common(q, k, v, s0, o, s_out, return_state):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d_k]")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    _require(q, "q", (B, H, T, dk), q.dtype, dev)
    _require(k, "k", (B, H, T, dk), q.dtype, dev)
    _require(v, "v", (B, H, T, dv), q.dtype, dev)
    if s0 is not None:
        _require(s0, "s0", (B, H, dv, dk), torch.float32, dev)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", (B, H, T, dv), q.dtype, dev)
    if s_out is None and return_state:
        s_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    elif s_out is not None:
        _require(s_out, "s_out", (B, H, dv, dk), torch.float32, dev)
    return (B, H, T, dk, dv), o, s_out


def la_chunk_fwd(q, k, v, log_gamma, chunk=64, s0=None, o=None, s_out=None, return_state=True,
                 workspace=None):
    """Retention with a fixed decay per head: S_t = gamma_h S_{t-1} + v_t k_t^T, o_t = S_t q_t.

    q, k [B,H,T,d_k], v [B,H,T,d_v] (bf16 or fp32); log_gamma [H] fp32. Returns (o, s_out).
    `workspace` (optional) is a device tensor of at least workspace_size() bytes."""
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(log_gamma, "log_gamma", (H,), torch.float32, q.device)
    ws, ws_bytes = _workspace(_native.LA_RETENTION, dims, chunk, q, workspace)
    lib = _native.load()
    _native.check(lib.la_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_gamma), _ptr(s0), _ptr(o),
                                   _ptr(s_out), B, H, T, dk, dv, chunk, _dtype_code(q), _ptr(ws), ws_bytes,
                                   _stream(q.device)))
    return o, s_out


def mamba2_chunk_fwd(q, k, v, log_alpha, chunk=64, s0=None, o=None, s_out=None, return_state=True,
                     workspace=None):
    """Scalar data-dependent decay: S_t = alpha_t S_{t-1} + v_t k_t^T, o_t = S_t q_t.

    log_alpha [B,H,T] fp32 (log of one gate per token and head). Returns (o, s_out)."""
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(log_alpha, "log_alpha", (B, H, T), torch.float32, q.device)
    ws, ws_bytes = _workspace(_native.LA_MAMBA2, dims, chunk, q, workspace)
    lib = _native.load()
    _native.check(lib.mamba2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(s0), _ptr(o),
                                       _ptr(s_out), B, H, T, dk, dv, chunk, _dtype_code(q), _ptr(ws), ws_bytes,
                                       _stream(q.device)))
    return o, s_out


def gla_chunk_fwd(q, k, v, log_alpha, chunk=64, s0=None, o=None, s_out=None, return_state=True,
                  workspace=None):
    """Gated linear attention: S_t = S_{t-1} Diag(alpha_t) + v_t k_t^T, o_t = S_t q_t.

    log_alpha [B,H,T,d_k] fp32 (log of the per-key-channel gates). Returns (o, s_out)."""
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(log_alpha, "log_alpha", (B, H, T, dk), torch.float32, q.device)
    ws, ws_bytes = _workspace(_native.LA_GLA, dims, chunk, q, workspace)
    lib = _native.load()
    _native.check(lib.gla_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(s0), _ptr(o),
                                    _ptr(s_out), B, H, T, dk, dv, chunk, _dtype_code(q), _ptr(ws), ws_bytes,
                                    _stream(q.device)))
    return o, s_out


def gdelta_chunk_fwd(q, k, v, log_alpha, beta, chunk=64, s0=None, o=None, s_out=None, return_state=True,
                     workspace=None):
    """Gated delta rule: S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.

    log_alpha, beta [B,H,T] fp32. Returns (o, s_out)."""
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(log_alpha, "log_alpha", (B, H, T), torch.float32, q.device)
    _require(beta, "beta", (B, H, T), torch.float32, q.device)
    ws, ws_bytes = _workspace(_native.LA_GDELTA, dims, chunk, q, workspace)
    lib = _native.load()
    _native.check(lib.gdelta_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(s0),
                                       _ptr(o), _ptr(s_out), B, H, T, dk, dv, chunk, _dtype_code(q),
                                       _ptr(ws), ws_bytes, _stream(q.device)))
    return o, s_out


def gla_chunk_fwd_fused(q, k, v, log_alpha, o_norm_weight, o_norm_bias=None, o_norm_eps=1e-5, chunk=64, s0=None,
                        o=None, s_out=None, return_state=True, workspace=None):
    """gla_chunk_fwd with GLA's output LayerNorm fused in: every output row (d_v values)
    centred, divided by sqrt(var + o_norm_eps), times ``o_norm_weight`` [d_v] fp32 plus
    ``o_norm_bias`` [d_v] fp32 (None: no shift). Returns (o, s_out); s_out is the memory."""
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(log_alpha, "log_alpha", (B, H, T, dk), torch.float32, q.device)
    _require(o_norm_weight, "o_norm_weight", (dv,), torch.float32, q.device)
    if o_norm_bias is not None:
        _require(o_norm_bias, "o_norm_bias", (dv,), torch.float32, q.device)
    ws, ws_bytes = _workspace(_native.LA_GLA, dims, chunk, q, workspace)
    lib = _native.load()
    _native.check(lib.gla_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(s0), _ptr(o), _ptr(s_out),
                                          _ptr(o_norm_weight), _ptr(o_norm_bias), float(o_norm_eps),
                                          _native.LA_FUSE_OUT_LAYERNORM, B, H, T, dk, dv, chunk, _dtype_code(q),
                                          _ptr(ws), ws_bytes, _stream(q.device)))
    return o, s_out


def _norm_fused(fn, variant, gate, gate_shape, q, k, v, o_norm_weight, o_norm_bias, o_norm_eps, norm, chunk, s0, o,
                s_out, return_state, workspace):
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(gate, "gate", gate_shape(B, H, T, dk), torch.float32, q.device)
    _require(o_norm_weight, "o_norm_weight", (dv,), torch.float32, q.device)
    if o_norm_bias is not None:
        _require(o_norm_bias, "o_norm_bias", (dv,), torch.float32, q.device)
    fuse = {"rms": _native.LA_FUSE_OUT_RMSNORM, "layer": _native.LA_FUSE_OUT_LAYERNORM}[norm]
    ws, ws_bytes = _workspace(variant, dims, chunk, q, workspace)
    lib = _native.load()
    _native.check(getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(s0), _ptr(o), _ptr(s_out),
                                   _ptr(o_norm_weight), _ptr(o_norm_bias), float(o_norm_eps), fuse, B, H, T, dk, dv,
                                   chunk, _dtype_code(q), _ptr(ws), ws_bytes, _stream(q.device)))
    return o, s_out


def la_chunk_fwd_fused(q, k, v, log_gamma, o_norm_weight, o_norm_bias=None, o_norm_eps=1e-5, norm="layer", chunk=64,
                       s0=None, o=None, s_out=None, return_state=True, workspace=None):
    """la_chunk_fwd with an output norm over each row of d_v values: ``norm="layer"`` (centred,
    divided by sqrt(var + eps), times ``o_norm_weight`` plus ``o_norm_bias`` or nothing) or
    ``norm="rms"`` (divided by sqrt(mean square + eps), times ``o_norm_weight``; no bias).
    Returns (o, s_out); s_out is the memory."""
    return _norm_fused("la_chunk_fwd_fused", _native.LA_RETENTION, log_gamma, lambda B, H, T, dk: (H,), q, k, v,
                       o_norm_weight, o_norm_bias, o_norm_eps, norm, chunk, s0, o, s_out, return_state, workspace)


def mamba2_chunk_fwd_fused(q, k, v, log_alpha, o_norm_weight, o_norm_bias=None, o_norm_eps=1e-5, norm="layer",
                           chunk=64, s0=None, o=None, s_out=None, return_state=True, workspace=None):
    """mamba2_chunk_fwd with an output norm, as la_chunk_fwd_fused."""
    return _norm_fused("mamba2_chunk_fwd_fused", _native.LA_MAMBA2, log_alpha, lambda B, H, T, dk: (B, H, T), q, k, v,
                       o_norm_weight, o_norm_bias, o_norm_eps, norm, chunk, s0, o, s_out, return_state, workspace)


NOALLOC_SCRATCH_BYTES = 96 << 20   # the fixed workspace of gdelta_chunk_fwd_noalloc, per device


def gdelta_chunk_fwd_noalloc(q, k, v, log_alpha, beta, chunk=64, s0=None, o=None, s_out=None, return_state=True):
    """gdelta_chunk_fwd whose workspace is the library's fixed per-device array of
    NOALLOC_SCRATCH_BYTES: with ``o`` passed in and ``s_out`` passed in (or
    ``return_state=False``), the call allocates nothing. Calls overlapping in time on one
    device race on that array."""
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(log_alpha, "log_alpha", (B, H, T), torch.float32, q.device)
    _require(beta, "beta", (B, H, T), torch.float32, q.device)
    lib = _native.load()
    _native.check(lib.gdelta_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(s0),
                                               _ptr(o), _ptr(s_out), B, H, T, dk, dv, chunk, _dtype_code(q),
                                               _stream(q.device)))
    return o, s_out


def gdelta_chunk_fwd_fused(q, k, v, log_alpha, beta, chunk=64, qk_silu_l2=True, o_norm_weight=None,
                           o_norm_eps=1e-6, s0=None, o=None, s_out=None, return_state=True, workspace=None):
    """gdelta_chunk_fwd with DeltaNet's feature map and output norm fused in: with
    ``qk_silu_l2`` q and k are the projections before SiLU + L2 normalisation; with an
    ``o_norm_weight`` [d_v] fp32 every output row is RMS-normalised and weighted."""
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    _require(log_alpha, "log_alpha", (B, H, T), torch.float32, q.device)
    _require(beta, "beta", (B, H, T), torch.float32, q.device)
    fuse = _native.LA_FUSE_QK_SILU_L2 if qk_silu_l2 else 0
    if o_norm_weight is not None:
        _require(o_norm_weight, "o_norm_weight", (dv,), torch.float32, q.device)
        fuse |= _native.LA_FUSE_OUT_RMSNORM
    ws, ws_bytes = _workspace(_native.LA_GDELTA_FUSED if qk_silu_l2 else _native.LA_GDELTA, dims, chunk, q,
                              workspace)
    lib = _native.load()
    _native.check(lib.gdelta_chunk_fwd_fused(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(s0),
                                             _ptr(o), _ptr(s_out), _ptr(o_norm_weight), float(o_norm_eps), fuse,
                                             B, H, T, dk, dv, chunk, _dtype_code(q), _ptr(ws), ws_bytes,
                                             _stream(q.device)))
    return o, s_out


def workspace_size(kind, B, H, T, dk, dv, chunk=64, dtype=torch.bfloat16):
    """Device workspace in bytes for a chunk entry point; kind in {"retention", "mamba2", "gla", "gdelta",
    "gdelta_fused"} ("gdelta_fused": gdelta_chunk_fwd_fused with the feature map fused in)."""
    variant = {"retention": _native.LA_RETENTION, "mamba2": _native.LA_MAMBA2, "gla": _native.LA_GLA,
               "gdelta": _native.LA_GDELTA, "gdelta_fused": _native.LA_GDELTA_FUSED}[kind]
    code = _native.LA_BF16 if dtype == torch.bfloat16 else _native.LA_F32
    return _native.workspace_size(variant, B, H, T, dk, dv, chunk, code)


def bwd_workspace_size(B, H, T, dk, dv, chunk=64, dtype=torch.bfloat16, gla=False, gdelta=False):
    """Device workspace in bytes for la_chunk_bwd and mamba2_chunk_bwd (``gla``: gla_chunk_bwd;
    ``gdelta``: gdelta_chunk_bwd)."""
    code = _native.LA_BF16 if dtype == torch.bfloat16 else _native.LA_F32
    return _native.bwd_workspace_size(B, H, T, dk, dv, chunk, code, gla, gdelta)


def la_recurrent_step(q, k, v, alpha, s, o=None):
    """One decode token, in place on s: S <- S Diag(alpha); S <- S + v k^T; o = S q.

    q, k [N,H,d_k], v [N,H,d_v] (bf16 or fp32); alpha [N,H,d_k] fp32; s [N,H,d_v,d_k] fp32."""
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    _require(k, "k", (N, H, dk), q.dtype, dev)
    _require(v, "v", (N, H, dv), q.dtype, dev)
    _require(alpha, "alpha", (N, H, dk), torch.float32, dev)
    _require(s, "s", (N, H, dv, dk), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", (N, H, dv), q.dtype, dev)
    lib = _native.load()
    _native.check(lib.la_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(s), _ptr(o),
                                        N, H, dk, dv, _dtype_code(q), _stream(dev)))
    return o


def gdelta_recurrent_step(q, k, v, alpha, beta, s, o=None):
    """One decode token of the gated delta rule, in place on s:
    S <- S [alpha (I - beta k k^T)] + beta v k^T; o = S q.

    q, k [N,H,d_k], v [N,H,d_v] (bf16 or fp32); alpha, beta [N,H] fp32; s [N,H,d_v,d_k] fp32."""
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    _require(k, "k", (N, H, dk), q.dtype, dev)
    _require(v, "v", (N, H, dv), q.dtype, dev)
    _require(alpha, "alpha", (N, H), torch.float32, dev)
    _require(beta, "beta", (N, H), torch.float32, dev)
    _require(s, "s", (N, H, dv, dk), torch.float32, dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", (N, H, dv), q.dtype, dev)
    lib = _native.load()
    _native.check(lib.gdelta_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s), _ptr(o),
                                            N, H, dk, dv, _dtype_code(q), _stream(dev)))
    return o


def _vla_readout(readout):
    codes = {"ratio": _native.LA_VLA_RATIO, "linear": _native.LA_VLA_LINEAR}
    if readout not in codes:
        raise ValueError(f"readout must be 'ratio' or 'linear', got {readout!r}")
    return codes[readout]


def vla_fwd(q, k, v, u, lambda0=1.0, a0=None, s0=None, n0=None, o=None, s_out=None, a_out=None, n_out=None,
            readout="ratio", return_state=True):
    """Variational linear attention over whole sequences: per token z = A u,
    A <- A - z z^T / (1 + u.z), a = A k^/|A k^|, S <- S + (v - S k^) a^T, then the readout:
    "ratio" (ELU+1 map phi on k and q, k^ = phi(k)/|phi(k)|, n <- n + (1 - n.k^) a,
    o = S phi(q) / (n.phi(q))) or "linear" (k^ = k/|k|, o = S q).

    q, k, u [B,H,T,d_k], v [B,H,T,d_v] (bf16 or fp32); A starts at a0 [B,H,d_k,d_k] fp32 or
    I / lambda0, S at s0 [B,H,d_v,d_k] fp32 or zeros, n at n0 [B,H,d_k] fp32 or zeros.
    Returns (o, s_out, a_out, n_out) (n_out None for the linear readout)."""
    code = _vla_readout(readout)
    dims, o, s_out = _chunk_common(q, k, v, s0, o, s_out, return_state)
    B, H, T, dk, dv = dims
    dev = q.device
    _require(u, "u", (B, H, T, dk), q.dtype, dev)
    if a0 is not None:
        _require(a0, "a0", (B, H, dk, dk), torch.float32, dev)
    if a_out is None and return_state:
        a_out = torch.empty((B, H, dk, dk), dtype=torch.float32, device=dev)
    elif a_out is not None:
        _require(a_out, "a_out", (B, H, dk, dk), torch.float32, dev)
    if code == _native.LA_VLA_RATIO:
        if n0 is not None:
            _require(n0, "n0", (B, H, dk), torch.float32, dev)
        if n_out is None and return_state:
            n_out = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
        elif n_out is not None:
            _require(n_out, "n_out", (B, H, dk), torch.float32, dev)
    else:
        n0 = n_out = None
    lib = _native.load()
    _native.check(lib.vla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(u), float(lambda0), _ptr(a0), _ptr(s0), _ptr(n0),
                              _ptr(o), _ptr(s_out), _ptr(a_out), _ptr(n_out), code, B, H, T, dk, dv, _dtype_code(q),
                              _stream(dev)))
    return o, s_out, a_out, n_out


def vla_recurrent_step(q, k, v, u, s, a, n=None, o=None, readout="ratio"):
    """One VLA decode token, in place on the memory s [N,H,d_v,d_k], the inverse penalty
    a [N,H,d_k,d_k] and (ratio readout) the denominator vector n [N,H,d_k] (fp32); q, k, u
    [N,H,d_k], v [N,H,d_v] (bf16 or fp32). Returns o."""
    code = _vla_readout(readout)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU")
    _require(k, "k", (N, H, dk), q.dtype, dev)
    _require(u, "u", (N, H, dk), q.dtype, dev)
    _require(v, "v", (N, H, dv), q.dtype, dev)
    _require(s, "s", (N, H, dv, dk), torch.float32, dev)
    _require(a, "a", (N, H, dk, dk), torch.float32, dev)
    if code == _native.LA_VLA_RATIO:
        _require(n, "n", (N, H, dk), torch.float32, dev)
    else:
        n = None
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(o, "o", (N, H, dv), q.dtype, dev)
    lib = _native.load()
    _native.check(lib.vla_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(s), _ptr(a), _ptr(n), _ptr(o), code,
                                         N, H, dk, dv, _dtype_code(q), _stream(dev)))
    return o


def _chunk_bwd(fn, q, k, v, gate, gate_shape, dout, s0, ds_out, chunk, want_ds0, workspace, gla=False):
    dims, _, _ = _chunk_common(q, k, v, s0, dout, None, False)
    B, H, T, dk, dv = dims
    dev = q.device
    _require(gate, "gate", gate_shape, torch.float32, dev)
    if ds_out is not None:
        _require(ds_out, "ds_out", (B, H, dv, dk), torch.float32, dev)
    dq, dk_ = torch.empty_like(q), torch.empty_like(k)
    dv_ = torch.empty_like(v)
    dgate = torch.empty(gate_shape, dtype=torch.float32, device=dev)
    ds0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_ds0 else None
    need = bwd_workspace_size(B, H, T, dk, dv, chunk, q.dtype, gla)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    _native.check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(s0), _ptr(dout), _ptr(ds_out), _ptr(dq), _ptr(dk_),
                     _ptr(dv_), _ptr(dgate), _ptr(ds0), B, H, T, dk, dv, chunk, _dtype_code(q), _ptr(workspace),
                     workspace.numel() * workspace.element_size(), _stream(dev)))
    return dq, dk_, dv_, dgate, ds0


def la_chunk_bwd(q, k, v, log_gamma, dout, s0=None, ds_out=None, chunk=64, want_ds0=True, workspace=None):
    """Gradients of la_chunk_fwd (bf16): given dout = dL/do and optionally ds_out = dL/dS_T, returns
    (dq, dk, dv, dlog_gamma [H], ds0 or None)."""
    return _chunk_bwd(_native.load().la_chunk_bwd, q, k, v, log_gamma, (q.shape[1],), dout, s0, ds_out, chunk,
                      want_ds0, workspace)


def gla_chunk_bwd(q, k, v, log_alpha, dout, s0=None, ds_out=None, chunk=64, want_ds0=True, workspace=None):
    """Gradients of gla_chunk_fwd (bf16): returns (dq, dk, dv, dlog_alpha [B,H,T,d_k], ds0 or None)."""
    return _chunk_bwd(_native.load().gla_chunk_bwd, q, k, v, log_alpha, tuple(q.shape), dout, s0, ds_out, chunk,
                      want_ds0, workspace, gla=True)


def gdelta_chunk_bwd(q, k, v, log_alpha, beta, dout, s0=None, ds_out=None, chunk=64, want_ds0=True, workspace=None):
    """Gradients of gdelta_chunk_fwd (bf16): given dout = dL/do and optionally ds_out = dL/dS_T,
    returns (dq, dk, dv, dlog_alpha [B,H,T], dbeta [B,H,T], ds0 or None)."""
    dims, _, _ = _chunk_common(q, k, v, s0, dout, None, False)
    B, H, T, dk, dv = dims
    dev = q.device
    _require(log_alpha, "log_alpha", (B, H, T), torch.float32, dev)
    _require(beta, "beta", (B, H, T), torch.float32, dev)
    if ds_out is not None:
        _require(ds_out, "ds_out", (B, H, dv, dk), torch.float32, dev)
    dq, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dla = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dbe = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    ds0 = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev) if want_ds0 else None
    need = bwd_workspace_size(B, H, T, dk, dv, chunk, q.dtype, gdelta=True)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the device of q")
    _native.check(_native.load().gdelta_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(s0), _ptr(dout), _ptr(ds_out), _ptr(dq),
        _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dbe), _ptr(ds0), B, H, T, dk, dv, chunk, _dtype_code(q),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return dq, dk_, dv_, dla, dbe, ds0


def mamba2_chunk_bwd(q, k, v, log_alpha, dout, s0=None, ds_out=None, chunk=64, want_ds0=True, workspace=None):
    """Gradients of mamba2_chunk_fwd (bf16): returns (dq, dk, dv, dlog_alpha [B,H,T], ds0 or None)."""
    return _chunk_bwd(_native.load().mamba2_chunk_bwd, q, k, v, log_alpha, tuple(q.shape[:3]), dout, s0, ds_out,
                      chunk, want_ds0, workspace)
