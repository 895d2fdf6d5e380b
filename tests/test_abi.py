"""The C-ABI library loads without a GPU, exports what ``include/glr.h`` declares,
and rejects bad arguments before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

from gated_linear_recurrences_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "glr.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:la_status|const char\*|int|size_t)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _native.load()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("la_chunk_fwd", "mamba2_chunk_fwd", "gla_chunk_fwd", "gdelta_chunk_fwd", "la_recurrent_step"):
        assert n in names
    assert set(names) == set(_native.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.la_version() >> 16 == 3        # 3.0: the VLA entry points take the readout and its denominator
    assert lib.la_version() & 0xFFFF >= 4     # 3.1: noalloc; 3.2: gla_chunk_fwd_fused; 3.3: gdelta_chunk_bwd;
    #                                           3.4: la_chunk_fwd_fused, mamba2_chunk_fwd_fused
    assert lib.la_status_str(0) == b"ok"
    assert lib.la_status_str(1) == b"invalid argument"
    assert lib.la_status_str(2) == b"unsupported shape"
    assert lib.la_status_str(3) == b"HIP launch error"


FAKE = 1 << 20          # aligned, never dereferenced: every call below fails validation first
MISALIGNED = FAKE + 4


def _chunk(lib, fn, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, s0=None, o=FAKE, s_out=None,
             B=1, H=1, T=8, dk=16, dv=16, chunk=16, dtype=1, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    P = ctypes.c_void_p
    if fn == "gdelta_chunk_fwd":
        return lib.gdelta_chunk_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["gate"]), P(a["beta"]), P(a["s0"]),
                                    P(a["o"]), P(a["s_out"]), a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                    a["chunk"], a["dtype"], P(a["ws"]), a["ws_bytes"], None)
    return getattr(lib, fn)(P(a["q"]), P(a["k"]), P(a["v"]), P(a["gate"]), P(a["s0"]), P(a["o"]),
                            P(a["s_out"]), a["B"], a["H"], a["T"], a["dk"], a["dv"], a["chunk"], a["dtype"],
                            P(a["ws"]), a["ws_bytes"], None)


VARIANT = {"la_chunk_fwd": _native.LA_RETENTION, "mamba2_chunk_fwd": _native.LA_MAMBA2,
           "gla_chunk_fwd": _native.LA_GLA, "gdelta_chunk_fwd": _native.LA_GDELTA}


def _ws(lib, variant, B=1, H=1, T=8, dk=16, dv=16, chunk=16, dtype=1):
    out = ctypes.c_size_t(12345)
    st = lib.la_chunk_workspace_size(variant, B, H, T, dk, dv, chunk, dtype, ctypes.byref(out))
    return st, out.value


def test_workspace_size_query(lib):
    # retention, the scalar decay and GLA in bf16, two-pass forward: one bf16 d_v x d_k memory
    # per (sequence, chunk). Retention and the scalar decay take the single-pass forward, with
    # no workspace, once B * H * d_v / 16 >= 128; GLA too at chunk 64 with d_k of 64 or 128.
    assert _ws(lib, _native.LA_GLA, B=4, H=8, T=2048, dk=128, dv=128, chunk=64) == (_native.LA_OK, 0)
    assert _ws(lib, _native.LA_GLA, B=4, H=4, T=100, dk=64, dv=128, chunk=64) == (_native.LA_OK, 0)
    assert _ws(lib, _native.LA_GLA, B=4, H=4, T=100, dk=32, dv=128, chunk=64) == (_native.LA_OK, 16 * 2 * 128 * 32 * 2)
    assert _ws(lib, _native.LA_GLA, B=2, H=4, T=100, dk=64, dv=128, chunk=64) == (_native.LA_OK, 8 * 2 * 128 * 64 * 2)
    assert _ws(lib, _native.LA_GLA, B=8, H=8, T=100, dk=16, dv=128, chunk=64) == (_native.LA_OK, 64 * 2 * 128 * 16 * 2)
    assert _ws(lib, _native.LA_GLA, B=8, H=8, T=100, dk=64, dv=128, chunk=32) == (_native.LA_OK, 64 * 4 * 128 * 64 * 2)
    for variant in (_native.LA_RETENTION, _native.LA_MAMBA2):
        assert _ws(lib, variant, B=4, H=8, T=2048, dk=128, dv=128, chunk=64) == (_native.LA_OK, 0)
        assert _ws(lib, variant, B=4, H=4, T=100, dk=64, dv=128, chunk=64) == (_native.LA_OK, 0)
        assert _ws(lib, variant, B=2, H=4, T=100, dk=64, dv=128, chunk=64) == (_native.LA_OK, 8 * 2 * 128 * 64 * 2)
        assert _ws(lib, variant, B=8, H=8, T=100, dk=64, dv=16, chunk=64) == (_native.LA_OK, 64 * 2 * 16 * 64 * 2)
    for variant in (_native.LA_RETENTION, _native.LA_MAMBA2, _native.LA_GLA):
        assert _ws(lib, variant, B=1, H=2, T=65, dk=32, dv=64, chunk=32) == (_native.LA_OK, 2 * 3 * 64 * 32 * 2)
        assert _ws(lib, variant, T=0) == (_native.LA_OK, 0)
        assert _ws(lib, variant, B=0) == (_native.LA_OK, 0)
        assert _ws(lib, variant, dtype=0) == (_native.LA_OK, 0)      # fp32 storage: one fused kernel
    # gated delta rule in bf16, each array rounded up to 256 bytes. Chunk 64 with d_k >= 32:
    # T_U (chunk x chunk bf16) and the cumulative gates per chunk (the mapped q and k as well
    # with the fused feature map); otherwise W, pseudo-values, cumulative gates and the memory
    def a256(x):
        return (x + 255) // 256 * 256

    for (B, H, T, dk, dv) in ((4, 16, 8192, 128, 128), (1, 3, 100, 32, 64), (2, 1, 64, 64, 16)):
        n = B * H * ((T + 63) // 64)
        want = a256(n * 64 * 64 * 2) + a256(n * 64 * 4)
        assert _ws(lib, _native.LA_GDELTA, B=B, H=H, T=T, dk=dk, dv=dv, chunk=64) == (_native.LA_OK, want)
        want += 2 * a256(n * 64 * dk * 2)
        assert _ws(lib, _native.LA_GDELTA_FUSED, B=B, H=H, T=T, dk=dk, dv=dv, chunk=64) == (_native.LA_OK, want)
    for (B, H, T, dk, dv, C) in ((1, 2, 65, 32, 64, 32), (1, 1, 40, 16, 16, 16), (2, 2, 100, 16, 64, 64)):
        n = B * H * ((T + C - 1) // C)
        want = a256(n * C * dk * 2) + a256(n * dv * C * 4) + a256(n * C * 4) + a256(n * dv * dk * 2)
        assert _ws(lib, _native.LA_GDELTA, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C) == (_native.LA_OK, want)
        # with the fused feature map the mapped keys are kept too
        want += a256(n * C * dk * 2)
        assert _ws(lib, _native.LA_GDELTA_FUSED, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C) == (_native.LA_OK, want)
    assert _ws(lib, _native.LA_GDELTA, T=0) == (_native.LA_OK, 0)
    assert _ws(lib, _native.LA_GDELTA, dtype=0) == (_native.LA_OK, 0)
    assert _ws(lib, 7)[0] == _native.LA_ERR_INVALID
    assert _ws(lib, 0, dk=24)[0] == _native.LA_ERR_UNSUPPORTED
    assert _ws(lib, 0, chunk=48)[0] == _native.LA_ERR_UNSUPPORTED
    assert _ws(lib, 0, T=-1)[0] == _native.LA_ERR_INVALID
    assert _ws(lib, 0, dtype=5)[0] == _native.LA_ERR_INVALID
    assert lib.la_chunk_workspace_size(0, 1, 1, 8, 16, 16, 16, 1, None) == _native.LA_ERR_INVALID


@pytest.mark.parametrize("fn", ["la_chunk_fwd", "mamba2_chunk_fwd", "gla_chunk_fwd", "gdelta_chunk_fwd"])
def test_chunk_workspace_validation(lib, fn):
    st, need = _ws(lib, VARIANT[fn], T=40, chunk=16)
    assert st == _native.LA_OK and need == (6400 if fn == "gdelta_chunk_fwd" else 3 * 16 * 16 * 2)
    assert _chunk(lib, fn, T=40, ws=None, q=None) == _native.LA_ERR_INVALID      # argument checks come first
    assert _chunk(lib, fn, T=40, ws=None) == _native.LA_ERR_INVALID
    assert b"workspace is NULL" in lib.la_last_error()
    assert _chunk(lib, fn, T=40, ws_bytes=need - 1) == _native.LA_ERR_INVALID
    assert b"workspace too small" in lib.la_last_error()
    assert _chunk(lib, fn, T=40, ws=MISALIGNED) == _native.LA_ERR_INVALID


@pytest.mark.parametrize("fn", ["la_chunk_fwd", "mamba2_chunk_fwd", "gla_chunk_fwd", "gdelta_chunk_fwd"])
def test_chunk_validation(lib, fn):
    assert _chunk(lib, fn, q=None) == _native.LA_ERR_INVALID
    assert b"q is NULL" in lib.la_last_error()
    assert _chunk(lib, fn, o=None) == _native.LA_ERR_INVALID
    assert _chunk(lib, fn, gate=None) == _native.LA_ERR_INVALID
    assert _chunk(lib, fn, v=MISALIGNED) == _native.LA_ERR_INVALID
    assert b"aligned" in lib.la_last_error()
    assert _chunk(lib, fn, s_out=MISALIGNED) == _native.LA_ERR_INVALID
    assert _chunk(lib, fn, T=-1) == _native.LA_ERR_INVALID
    assert _chunk(lib, fn, chunk=0) == _native.LA_ERR_INVALID
    assert _chunk(lib, fn, dtype=7) == _native.LA_ERR_INVALID
    assert _chunk(lib, fn, dk=24) == _native.LA_ERR_UNSUPPORTED
    assert _chunk(lib, fn, dv=256) == _native.LA_ERR_UNSUPPORTED
    assert _chunk(lib, fn, chunk=48) == _native.LA_ERR_UNSUPPORTED
    if fn == "gdelta_chunk_fwd":
        assert _chunk(lib, fn, beta=None) == _native.LA_ERR_INVALID
    # T == 0 launches kernels that read retention's per-head decay (and write s_out): the decay is
    # required whenever there are heads; the per-token gates only when there are tokens
    if fn == "la_chunk_fwd":
        assert _chunk(lib, fn, T=0, gate=None) == _native.LA_ERR_INVALID
        assert b"log_gamma is NULL" in lib.la_last_error()
    # nothing to do: no pointer is needed and nothing is launched
    assert _chunk(lib, fn, B=0, q=None, k=None, v=None, o=None, gate=None, beta=None) == _native.LA_OK
    assert _chunk(lib, fn, H=0, q=None, k=None, v=None, o=None, gate=None, beta=None) == _native.LA_OK


def test_decode_validation(lib):
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, s=FAKE, o=FAKE, N=4, H=2, dk=128, dv=128, dtype=1)
        a.update(kw)
        return lib.la_recurrent_step(P(a["q"]), P(a["k"]), P(a["v"]), P(a["alpha"]), P(a["s"]), P(a["o"]),
                                     a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)

    assert call(s=None) == _native.LA_ERR_INVALID
    assert call(alpha=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(N=-1) == _native.LA_ERR_INVALID
    assert call(dk=48) == _native.LA_ERR_UNSUPPORTED
    assert call(dtype=3) == _native.LA_ERR_INVALID
    assert call(N=0, q=None, k=None, v=None, alpha=None, s=None, o=None) == _native.LA_OK


def test_gdelta_decode_validation(lib):
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, s=FAKE, o=FAKE, N=4, H=2, dk=128, dv=128, dtype=1)
        a.update(kw)
        return lib.gdelta_recurrent_step(P(a["q"]), P(a["k"]), P(a["v"]), P(a["alpha"]), P(a["beta"]), P(a["s"]),
                                         P(a["o"]), a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)

    assert call(beta=None) == _native.LA_ERR_INVALID
    assert b"beta is NULL" in lib.la_last_error()
    assert call(s=None) == _native.LA_ERR_INVALID
    assert call(alpha=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(N=-1) == _native.LA_ERR_INVALID
    assert call(dk=48) == _native.LA_ERR_UNSUPPORTED
    assert call(dtype=3) == _native.LA_ERR_INVALID
    assert call(N=0, q=None, k=None, v=None, alpha=None, beta=None, s=None, o=None) == _native.LA_OK


def test_gdelta_fused_validation(lib):
    P = ctypes.c_void_p

    def call(fuse, weight=FAKE, eps=1e-6, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, o=FAKE, B=1, H=1, T=8, dk=16, dv=16, chunk=16)
        a.update(kw)
        return lib.gdelta_chunk_fwd_fused(P(a["q"]), P(a["k"]), P(a["v"]), P(a["gate"]), P(a["beta"]), None,
                                          P(a["o"]), None, P(weight), eps, fuse, a["B"], a["H"], a["T"], a["dk"],
                                          a["dv"], a["chunk"], 1, P(FAKE), 1 << 30, None)

    assert call(4) == _native.LA_ERR_INVALID
    assert b"unknown fuse flag" in lib.la_last_error()
    assert call(_native.LA_FUSE_OUT_RMSNORM, weight=None) == _native.LA_ERR_INVALID
    assert b"o_norm_weight is NULL" in lib.la_last_error()
    assert call(_native.LA_FUSE_OUT_RMSNORM, weight=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_OUT_RMSNORM, eps=-1.0) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_OUT_RMSNORM, eps=float("nan")) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_QK_SILU_L2, q=None) == _native.LA_ERR_INVALID
    assert call(3, B=0, q=None, k=None, v=None, o=None, gate=None, beta=None, weight=None) == _native.LA_OK


def test_gla_fused_validation(lib):
    P = ctypes.c_void_p

    def call(fuse, weight=FAKE, bias=None, eps=1e-5, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, o=FAKE, B=1, H=1, T=8, dk=16, dv=16, chunk=16)
        a.update(kw)
        return lib.gla_chunk_fwd_fused(P(a["q"]), P(a["k"]), P(a["v"]), P(a["gate"]), None, P(a["o"]), None,
                                       P(weight), P(bias), eps, fuse, a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                       a["chunk"], 1, P(FAKE), 1 << 30, None)

    for flag in (_native.LA_FUSE_QK_SILU_L2, _native.LA_FUSE_OUT_RMSNORM, 8):
        assert call(flag) == _native.LA_ERR_INVALID
        assert b"fuse flag" in lib.la_last_error()
    assert call(_native.LA_FUSE_OUT_LAYERNORM, weight=None) == _native.LA_ERR_INVALID
    assert b"o_norm_weight is NULL" in lib.la_last_error()
    assert call(_native.LA_FUSE_OUT_LAYERNORM, weight=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_OUT_LAYERNORM, bias=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_OUT_LAYERNORM, eps=-1.0) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_OUT_LAYERNORM, eps=float("nan")) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_OUT_LAYERNORM, gate=None) == _native.LA_ERR_INVALID
    assert call(_native.LA_FUSE_OUT_LAYERNORM, B=0, q=None, k=None, v=None, o=None, gate=None,
                weight=None) == _native.LA_OK


@pytest.mark.parametrize("fn", ["la_chunk_fwd_fused", "mamba2_chunk_fwd_fused"])
def test_norm_fused_validation(lib, fn):
    P = ctypes.c_void_p

    def call(fuse, weight=FAKE, bias=None, eps=1e-5, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, o=FAKE, B=1, H=1, T=8, dk=16, dv=16, chunk=16)
        a.update(kw)
        return getattr(lib, fn)(P(a["q"]), P(a["k"]), P(a["v"]), P(a["gate"]), None, P(a["o"]), None,
                                P(weight), P(bias), eps, fuse, a["B"], a["H"], a["T"], a["dk"], a["dv"],
                                a["chunk"], 1, P(FAKE), 1 << 30, None)

    for flag in (0, _native.LA_FUSE_QK_SILU_L2, _native.LA_FUSE_OUT_RMSNORM | _native.LA_FUSE_OUT_LAYERNORM, 8):
        assert call(flag) == _native.LA_ERR_INVALID
        assert b"fuse must be" in lib.la_last_error()
    for flag in (_native.LA_FUSE_OUT_RMSNORM, _native.LA_FUSE_OUT_LAYERNORM):
        assert call(flag, weight=None) == _native.LA_ERR_INVALID
        assert b"o_norm_weight is NULL" in lib.la_last_error()
        assert call(flag, weight=MISALIGNED) == _native.LA_ERR_INVALID
        assert call(flag, eps=-1.0) == _native.LA_ERR_INVALID
        assert call(flag, eps=float("nan")) == _native.LA_ERR_INVALID
        assert call(flag, gate=None) == _native.LA_ERR_INVALID
        assert call(flag, B=0, q=None, k=None, v=None, o=None, gate=None, weight=None) == _native.LA_OK
    assert call(_native.LA_FUSE_OUT_RMSNORM, bias=FAKE) == _native.LA_ERR_INVALID
    assert b"no bias" in lib.la_last_error()
    assert call(_native.LA_FUSE_OUT_LAYERNORM, bias=MISALIGNED) == _native.LA_ERR_INVALID


def test_backward_validation(lib):
    P = ctypes.c_void_p

    def call(fn="la_chunk_bwd", ws_bytes=1 << 30, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, s0=None, dout=FAKE, ds_out=None, dq=FAKE, dk=FAKE, dv=FAKE,
                 dgate=FAKE, ds0=None, B=1, H=1, T=8, dk_=16, dv_=16, chunk=16, dtype=1, ws=FAKE)
        a.update(kw)
        return getattr(lib, fn)(P(a["q"]), P(a["k"]), P(a["v"]), P(a["gate"]), P(a["s0"]), P(a["dout"]),
                                P(a["ds_out"]), P(a["dq"]), P(a["dk"]), P(a["dv"]), P(a["dgate"]), P(a["ds0"]),
                                a["B"], a["H"], a["T"], a["dk_"], a["dv_"], a["chunk"], a["dtype"], P(a["ws"]),
                                ws_bytes, None)

    for fn in ("la_chunk_bwd", "mamba2_chunk_bwd", "gla_chunk_bwd"):
        assert call(fn, dtype=0) == _native.LA_ERR_UNSUPPORTED
        assert b"bf16" in lib.la_last_error()
        assert call(fn, dout=None) == _native.LA_ERR_INVALID
        assert b"dout is NULL" in lib.la_last_error()
        assert call(fn, dgate=None) == _native.LA_ERR_INVALID
        assert call(fn, ds_out=MISALIGNED) == _native.LA_ERR_INVALID
        assert call(fn, ws=None) == _native.LA_ERR_INVALID
        assert call(fn, ws_bytes=16) == _native.LA_ERR_INVALID
        assert b"workspace too small" in lib.la_last_error()
        assert call(fn, dk_=24) == _native.LA_ERR_UNSUPPORTED
        if fn == "la_chunk_bwd":
            assert call(fn, T=0, gate=None) == _native.LA_ERR_INVALID
        assert call(fn, B=0, q=None, k=None, v=None, gate=None, dout=None, dq=None, dk=None, dv=None,
                    dgate=None, ws=None) == _native.LA_OK


def test_gdelta_backward_validation(lib):
    P = ctypes.c_void_p

    def call(ws_bytes=1 << 30, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, s0=None, dout=FAKE, ds_out=None, dq=FAKE, dk=FAKE,
                 dv=FAKE, dgate=FAKE, dbeta=FAKE, ds0=None, B=1, H=1, T=8, dk_=16, dv_=16, chunk=16, dtype=1, ws=FAKE)
        a.update(kw)
        return lib.gdelta_chunk_bwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["gate"]), P(a["beta"]), P(a["s0"]),
                                    P(a["dout"]), P(a["ds_out"]), P(a["dq"]), P(a["dk"]), P(a["dv"]), P(a["dgate"]),
                                    P(a["dbeta"]), P(a["ds0"]), a["B"], a["H"], a["T"], a["dk_"], a["dv_"], a["chunk"],
                                    a["dtype"], P(a["ws"]), ws_bytes, None)

    assert call(dtype=0) == _native.LA_ERR_UNSUPPORTED
    assert b"bf16" in lib.la_last_error()
    assert call(beta=None) == _native.LA_ERR_INVALID
    assert b"beta is NULL" in lib.la_last_error()
    assert call(dbeta=None) == _native.LA_ERR_INVALID
    assert b"dbeta is NULL" in lib.la_last_error()
    assert call(dout=None) == _native.LA_ERR_INVALID
    assert call(dgate=None) == _native.LA_ERR_INVALID
    assert call(ds0=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(ws_bytes=16) == _native.LA_ERR_INVALID
    assert b"workspace too small" in lib.la_last_error()
    assert call(chunk=8) == _native.LA_ERR_UNSUPPORTED
    assert call(B=0, q=None, k=None, v=None, gate=None, beta=None, dout=None, dq=None, dk=None, dv=None,
                dgate=None, dbeta=None, ws=None) == _native.LA_OK
    # the workspace formula of the header (C = 64, d = 128, N = 4 * 16 * 128 chunks)
    def a256(x):
        return (x + 255) // 256 * 256
    need = ctypes.c_size_t(0)
    assert lib.gdelta_chunk_bwd_workspace_size(4, 16, 8192, 128, 128, 64, 1, ctypes.byref(need)) == _native.LA_OK
    N, C, d = 4 * 16 * 128, 64, 128
    want = (2 * a256(N * C * C * 2) + a256(N * C * 4) + a256(N * d * C * 2) + 2 * a256(N * d * d * 2)
            + 3 * a256(N * d * d * 2) + 3 * a256(N * C * d * 2)
            + a256(min(N, 512) * (6 * C * d + 3 * C * d + 6 * C * C + d * d) * 4))
    assert need.value == want


def test_backward_workspace_size(lib):
    def a256(x):
        return (x + 255) // 256 * 256

    out = ctypes.c_size_t(0)
    assert lib.la_chunk_bwd_workspace_size(4, 8, 2048, 128, 128, 64, 1, ctypes.byref(out)) == _native.LA_OK
    n = 4 * 8 * 32
    assert out.value == 2 * a256(n * 128 * 128 * 2) + a256(32 * 128 * 128 * 4) + a256(32 * 2048 * 4)
    assert lib.la_chunk_bwd_workspace_size(4, 8, 2048, 128, 128, 64, 0, ctypes.byref(out)) == _native.LA_ERR_UNSUPPORTED
    assert lib.la_chunk_bwd_workspace_size(0, 8, 2048, 128, 128, 64, 1, ctypes.byref(out)) == _native.LA_OK
    assert out.value == 0


def test_vla_validation(lib):
    P = ctypes.c_void_p

    def call(lam=1.0, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, a0=None, s0=None, n0=None, o=FAKE, s_out=None, a_out=None,
                 n_out=None, readout=_native.LA_VLA_RATIO, B=2, H=2, T=8, dk=64, dv=64, dtype=1)
        a.update(kw)
        return lib.vla_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["u"]), lam, P(a["a0"]), P(a["s0"]), P(a["n0"]),
                           P(a["o"]), P(a["s_out"]), P(a["a_out"]), P(a["n_out"]), a["readout"], a["B"], a["H"],
                           a["T"], a["dk"], a["dv"], a["dtype"], None)

    assert call(readout=2) == _native.LA_ERR_INVALID
    assert b"unknown readout" in lib.la_last_error()
    assert call(n0=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(n_out=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(u=None) == _native.LA_ERR_INVALID
    assert b"u is NULL" in lib.la_last_error()
    assert call(lam=0.0) == _native.LA_ERR_INVALID
    assert b"lambda0" in lib.la_last_error()
    assert call(lam=float("nan")) == _native.LA_ERR_INVALID
    assert call(lam=float("inf")) == _native.LA_ERR_INVALID
    assert call(a0=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(s_out=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(T=-1) == _native.LA_ERR_INVALID
    assert call(dk=48) == _native.LA_ERR_UNSUPPORTED
    assert call(dv=256) == _native.LA_ERR_UNSUPPORTED
    assert call(dtype=2) == _native.LA_ERR_INVALID
    assert call(B=0, q=None, k=None, v=None, u=None, o=None) == _native.LA_OK
    assert call(lam=0.0, B=0, q=None, k=None, v=None, u=None, o=None, a0=FAKE) == _native.LA_OK


def test_vla_decode_validation(lib):
    P = ctypes.c_void_p

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, s=FAKE, a=FAKE, n=FAKE, o=FAKE, readout=_native.LA_VLA_RATIO, N=4,
                 H=2, dk=128, dv=128, dtype=1)
        a.update(kw)
        return lib.vla_recurrent_step(P(a["q"]), P(a["k"]), P(a["v"]), P(a["u"]), P(a["s"]), P(a["a"]), P(a["n"]),
                                      P(a["o"]), a["readout"], a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)

    assert call(n=None) == _native.LA_ERR_INVALID                    # the ratio readout carries n
    assert b"n is NULL" in lib.la_last_error()
    assert call(readout=-1) == _native.LA_ERR_INVALID
    assert call(a=None) == _native.LA_ERR_INVALID
    assert b"a is NULL" in lib.la_last_error()
    assert call(u=MISALIGNED) == _native.LA_ERR_INVALID
    assert call(H=-1) == _native.LA_ERR_INVALID
    assert call(dv=8) == _native.LA_ERR_UNSUPPORTED
    assert call(N=0, q=None, k=None, v=None, u=None, s=None, a=None, o=None) == _native.LA_OK


def test_gla_backward_workspace_size(lib):
    def a256(x):
        return (x + 255) // 256 * 256

    out = ctypes.c_size_t(0)
    assert lib.gla_chunk_bwd_workspace_size(8, 16, 4096, 128, 128, 64, 1, ctypes.byref(out)) == _native.LA_OK
    n = 8 * 16 * 64
    assert out.value == 2 * a256(n * 128 * 128 * 2) + a256(128 * 128 * 128 * 4)
    assert lib.gla_chunk_bwd_workspace_size(1, 1, 8, 16, 16, 16, 0, ctypes.byref(out)) == _native.LA_ERR_UNSUPPORTED


def test_noalloc_validation(lib):
    """The no-allocation gated delta entry point checks every argument, then the size of the
    workspace its shape needs against its fixed array, before it touches a device."""
    fn = lib.gdelta_chunk_fwd_noalloc
    p = ctypes.c_void_p(4096)

    def call(q=p, beta=p, B=2, H=2, T=100, dk=64, dv=64, chunk=64, dtype=_native.LA_BF16):
        return fn(q, p, p, p, beta, None, p, None, B, H, T, dk, dv, chunk, dtype, None)

    assert call(q=None) == _native.LA_ERR_INVALID and b"q is NULL" in lib.la_last_error()
    assert call(beta=None) == _native.LA_ERR_INVALID and b"beta" in lib.la_last_error()
    assert call(q=ctypes.c_void_p(4100)) == _native.LA_ERR_INVALID
    assert call(T=-1) == _native.LA_ERR_INVALID
    assert call(dk=48) == _native.LA_ERR_UNSUPPORTED
    assert call(chunk=8) == _native.LA_ERR_UNSUPPORTED
    # B4 H16 T8192 d128 (66 MiB) fits the 96 MiB array; 16 x 16 x 8192 tokens at d 128 (264 MiB) do not
    need = ctypes.c_size_t(0)
    assert lib.la_chunk_workspace_size(_native.LA_GDELTA, 4, 16, 8192, 128, 128, 64, _native.LA_BF16,
                                       ctypes.byref(need)) == _native.LA_OK
    assert need.value <= 96 << 20
    assert call(B=16, H=16, T=8192, dk=128, dv=128) == _native.LA_ERR_UNSUPPORTED
    assert b"exceeds" in lib.la_last_error()
    # B == 0 is a no-op that needs no device
    assert call(B=0) == _native.LA_OK
