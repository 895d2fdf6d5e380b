"""ctypes loader for ``libglr.so`` (the C ABI declared in ``include/glr.h``).

The library must have been built in-tree (``gated_linear_recurrences_amd.build``);
there is no fallback path: loading fails loudly when it is missing.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libglr.so")

LA_OK, LA_ERR_INVALID, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
LA_F32, LA_BF16 = 0, 1
LA_RETENTION, LA_GLA, LA_GDELTA, LA_MAMBA2, LA_GDELTA_FUSED = 0, 1, 2, 3, 4
LA_FUSE_QK_SILU_L2, LA_FUSE_OUT_RMSNORM, LA_FUSE_OUT_LAYERNORM = 1, 2, 4
LA_VLA_RATIO, LA_VLA_LINEAR = 0, 1

EXPORTED = (
    "la_chunk_workspace_size",
    "la_chunk_fwd",
    "mamba2_chunk_fwd",
    "gla_chunk_fwd",
    "gdelta_chunk_fwd",
    "gdelta_chunk_fwd_fused",
    "gla_chunk_fwd_fused",
    "la_chunk_fwd_fused",
    "mamba2_chunk_fwd_fused",
    "gdelta_chunk_fwd_noalloc",
    "la_recurrent_step",
    "gdelta_recurrent_step",
    "la_chunk_bwd_workspace_size",
    "la_chunk_bwd",
    "mamba2_chunk_bwd",
    "gla_chunk_bwd_workspace_size",
    "gla_chunk_bwd",
    "gdelta_chunk_bwd_workspace_size",
    "gdelta_chunk_bwd",
    "vla_fwd",
    "vla_recurrent_step",
    "la_status_str",
    "la_last_error",
    "la_version",
)

_lib = None


class GLRError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def load():
    """Load (once) and return the library with its argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m gated_linear_recurrences_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    chunk = [P, P, P, F, F, P, F, I, I, I, I, I, I, I, P, Z, P]
    lib.la_chunk_fwd.argtypes = chunk
    lib.gla_chunk_fwd.argtypes = chunk
    lib.mamba2_chunk_fwd.argtypes = chunk
    lib.gdelta_chunk_fwd.argtypes = [P, P, P, F, F, F, P, F, I, I, I, I, I, I, I, P, Z, P]
    lib.gdelta_chunk_fwd_fused.argtypes = [P, P, P, F, F, F, P, F, F, ctypes.c_float, I,
                                           I, I, I, I, I, I, I, P, Z, P]
    lib.gla_chunk_fwd_fused.argtypes = [P, P, P, F, F, P, F, F, F, ctypes.c_float, I, I, I, I, I, I, I, I, P, Z, P]
    lib.la_chunk_fwd_fused.argtypes = lib.gla_chunk_fwd_fused.argtypes
    lib.mamba2_chunk_fwd_fused.argtypes = lib.gla_chunk_fwd_fused.argtypes
    lib.gdelta_chunk_fwd_noalloc.argtypes = [P, P, P, F, F, F, P, F, I, I, I, I, I, I, I, P]
    lib.la_chunk_workspace_size.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.la_chunk_workspace_size.restype = ctypes.c_int
    lib.la_recurrent_step.argtypes = [P, P, P, F, F, P, I, I, I, I, I, P]
    lib.gdelta_recurrent_step.argtypes = [P, P, P, F, F, F, P, I, I, I, I, I, P]
    bwd = [P, P, P, F, F, P, F, P, P, P, F, F, I, I, I, I, I, I, I, P, Z, P]
    lib.la_chunk_bwd.argtypes = bwd
    lib.mamba2_chunk_bwd.argtypes = bwd
    lib.gla_chunk_bwd.argtypes = bwd
    lib.gla_chunk_bwd_workspace_size.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.gla_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.gdelta_chunk_bwd.argtypes = [P, P, P, F, F, F, P, F, P, P, P, F, F, F, I, I, I, I, I, I, I, P, Z, P]
    lib.gdelta_chunk_bwd.restype = ctypes.c_int
    lib.gdelta_chunk_bwd_workspace_size.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdelta_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.la_chunk_bwd_workspace_size.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.la_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.vla_fwd.argtypes = [P, P, P, P, ctypes.c_float, F, F, F, P, F, F, F, I, I, I, I, I, I, I, P]
    lib.vla_recurrent_step.argtypes = [P, P, P, P, F, F, F, P, I, I, I, I, I, I, P]
    for name in ("la_chunk_fwd", "mamba2_chunk_fwd", "gla_chunk_fwd", "gdelta_chunk_fwd", "gdelta_chunk_fwd_fused",
                 "gdelta_chunk_fwd_noalloc", "gla_chunk_fwd_fused", "la_chunk_fwd_fused",
                 "mamba2_chunk_fwd_fused", "la_recurrent_step", "gdelta_recurrent_step", "la_chunk_bwd", "mamba2_chunk_bwd", "gla_chunk_bwd", "gdelta_chunk_bwd", "vla_fwd",
                 "vla_recurrent_step"):
        getattr(lib, name).restype = ctypes.c_int
    lib.la_status_str.argtypes = [ctypes.c_int]
    lib.la_status_str.restype = ctypes.c_char_p
    lib.la_last_error.argtypes = []
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_version.argtypes = []
    lib.la_version.restype = ctypes.c_int
    _lib = lib
    return lib


def workspace_size(variant, B, H, T, dk, dv, chunk, dtype):
    """Bytes of device workspace a chunk entry point needs for these sizes."""
    lib = load()
    out = ctypes.c_size_t(0)
    check(lib.la_chunk_workspace_size(variant, B, H, T, dk, dv, chunk, dtype, ctypes.byref(out)))
    return out.value


def check(status):
    """Raise GLRError for a non-OK status, with the library's message."""
    if status != LA_OK:
        lib = load()
        msg = lib.la_status_str(status).decode()
        detail = lib.la_last_error().decode()
        raise GLRError(status, f"{msg}: {detail}")


def bwd_workspace_size(B, H, T, dk, dv, chunk, dtype, gla=False, gdelta=False):
    """Bytes of device workspace the backward entry points need for these sizes (``gla``:
    gla_chunk_bwd's; ``gdelta``: gdelta_chunk_bwd's)."""
    lib = load()
    out = ctypes.c_size_t(0)
    fn = (lib.gdelta_chunk_bwd_workspace_size if gdelta else
          lib.gla_chunk_bwd_workspace_size if gla else lib.la_chunk_bwd_workspace_size)
    check(fn(B, H, T, dk, dv, chunk, dtype, ctypes.byref(out)))
    return out.value
