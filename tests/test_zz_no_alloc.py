"""gdelta_chunk_fwd_noalloc (the gated delta rule with its workspace in the library's fixed
per-device array) against gdelta_chunk_fwd with a caller-owned workspace, through the C ABI:
the same kernels on the same inputs, so outputs and final memories must agree bit for bit.
Each case makes two calls in a row, the second smaller, so the second runs on an array that
still holds the first call's contents."""

import numpy as np
import pytest
import torch

from gated_linear_recurrences_amd import api, synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _t(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def _pair(B, H, T, d, chunk, seed, state):
    w = synthetic.gdelta_inputs(B, H, T, d, d, chunk=chunk, dtype="bf16", seed=seed, with_state=state)
    args = (_t(w.q, torch.bfloat16), _t(w.k, torch.bfloat16), _t(w.v, torch.bfloat16), _t(w.log_alpha), _t(w.beta))
    s0 = _t(w.s0) if state else None
    o_ref, s_ref = api.gdelta_chunk_fwd(*args, chunk=chunk, s0=s0)
    o = torch.full_like(o_ref, float("nan"))
    s = torch.full_like(s_ref, float("nan"))
    api.gdelta_chunk_fwd_noalloc(*args, chunk=chunk, s0=s0, o=o, s_out=s)
    torch.cuda.synchronize()
    label = f"B{B} H{H} T{T} d{d} chunk {chunk} state={state}"
    print(f"noalloc {label}: max|do|={float((o.float() - o_ref.float()).abs().max()):.3e}", flush=True)
    assert torch.equal(o, o_ref), label
    assert torch.equal(s, s_ref), label


@pytest.mark.parametrize("chunk", [64, 32])
def test_noalloc_matches_the_workspace_entry_point(chunk):
    # the larger call first (several chunks per head and a ragged tail), then a smaller one
    _pair(2, 8, 2000, 128, chunk, seed=91, state=True)
    _pair(1, 3, 130, 64, chunk, seed=92, state=False)


def test_noalloc_rejects_a_shape_beyond_its_array():
    q = torch.zeros((16, 16, 8192, 128), dtype=torch.bfloat16, device=DEV)
    la = torch.zeros((16, 16, 8192), dtype=torch.float32, device=DEV)
    o = torch.empty_like(q)
    with pytest.raises(RuntimeError, match="exceeds"):
        api.gdelta_chunk_fwd_noalloc(q, q, q, la, la, chunk=64, o=o, return_state=False)
