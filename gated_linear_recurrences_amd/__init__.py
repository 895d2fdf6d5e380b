"""Gated linear recurrences on MI355X (gfx950): retention, the scalar data-dependent
decay, gated linear attention and the gated delta rule in chunkwise form, plus a
single-token decode step (per-channel gate or gated delta rule), the backward of
retention, the scalar decay and GLA, and variational linear attention (whole sequences and
decode).

The computation lives in the HIP library ``libglr.so`` (C ABI in ``include/glr.h``);
``api`` is its thin PyTorch binding with the same entry-point names.
"""

from .api import (la_chunk_fwd, mamba2_chunk_fwd, gla_chunk_fwd, gdelta_chunk_fwd,  # noqa: F401
                  gdelta_chunk_fwd_fused, la_chunk_bwd, mamba2_chunk_bwd, gla_chunk_bwd, la_recurrent_step,
                  gdelta_recurrent_step, vla_fwd, vla_recurrent_step, workspace_size,
                  bwd_workspace_size)

__all__ = ["la_chunk_fwd", "mamba2_chunk_fwd", "gla_chunk_fwd", "gdelta_chunk_fwd", "gdelta_chunk_fwd_fused",
           "la_chunk_bwd", "mamba2_chunk_bwd", "gla_chunk_bwd", "la_recurrent_step", "gdelta_recurrent_step",
           "vla_fwd", "vla_recurrent_step", "workspace_size", "bwd_workspace_size"]
