#!/usr/bin/env python3
"""Throughput of the chunked forward on one MI355X, with its roofline and the CPU oracle beside it.

A step is one call of the chunked forward - every stage of the hot path (the
memory carried from chunk to chunk, the decayed triangle, P V, the memory
readout, the stores), which at this size runs as one single-pass kernel (the
memory stays on chip; smaller batches take a state pass and an output pass) -
over one batch of the multi-scale retention workload: B=4,
H=8, T=2048, d_k=d_v=128, bf16 q/k/v ~ N(0,1)/sqrt(128), per-head decay
1 - 2^(-5-h), chunk 64, fp32 memory. Inputs are resident in HBM before timing;
five input sets are rotated so the 256 MB Infinity Cache cannot serve them.

Printed: one JSON line. ``value`` is tokens/s (B*H*T per second); ``roofline``
prices the call (its kernel, timed with HIP events on the launching stream around
one HIP-graph replay of the timed steps, so that host launches do not pace it)
against HBM with the algorithmic bytes of the method (q, k, v read, o and the
final memory written); ``traffic`` is the HBM traffic the counters measured for
one call; ``mfma`` gives the same run against the dense bf16
MFMA peak; ``cpu_baseline`` times the fp64 oracle on the host; ``others``
reports the per-channel-gate (GLA), gated-delta, scalar data-dependent decay
and decode (per-channel gate, gated delta rule) workloads measured the same way,
the gated delta rule with its feature map and output norm fused in, the
backward of the retention and scalar-decay workloads (beside their forward), and
variational linear attention (whole sequences, and decode).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-others] [--no-cpu]
    python bench.py --copy-calibration MB --steps K      (plain copy, for counter scaling)
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
    python bench.py --kernel-traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
    python bench.py --trace-table TRACE_DIR
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 (256 CU x 2.4 GHz x 4096 flop/clk)
N_SETS = 5                      # rotated input sets (> 256 MB Infinity Cache for the retention batch)

MAIN = "retention_b4h8_t2048_d128"


def algorithmic_counts(kind, B, H, T, d, chunk, elem_bytes=2):
    """Algorithmic flops and HBM bytes of one chunked-forward launch.

    Bytes: read q, k, v (and the gates), write o and the final memory.
    Flops per token-head (chunk C, head size d): retention, the scalar decay and GLA 4Cd + 4d^2
    (q.k^T and P.V over the C x C block, S q and k^T v); the gated delta rule
    8Cd + 6d^2 + 2C^2/3 (K K^T, Q K^T, T.R for W and U0, P.U, W S^T, Q S^T,
    U^T K and the triangular solve)."""
    th = B * H * T
    tok_bytes = 4 * d * elem_bytes
    gate_bytes = {"retention": 0, "mamba2": 4, "gla": 4 * d, "gdelta": 8}[kind]
    state_bytes = B * H * d * d * 4
    bytes_ = th * (tok_bytes + gate_bytes) + state_bytes
    if kind == "gdelta":
        flops = th * (8 * chunk * d + 6 * d * d + 2 * chunk * chunk / 3)
    else:
        flops = th * (4 * chunk * d + 4 * d * d)
    return flops, bytes_


def upload(w, torch, dev):
    def t(x, dt=torch.float32):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(dt).contiguous()
    st = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    d = {"q": t(w.q, st), "k": t(w.k, st), "v": t(w.v, st)}
    if w.log_gamma is not None:
        d["log_gamma"] = t(w.log_gamma)
    if w.log_alpha is not None:
        d["log_alpha"] = t(w.log_alpha)
    if w.beta is not None:
        d["beta"] = t(w.beta)
    return d


def make_call(kind, api, bufs, chunk, torch):
    q = bufs["q"]
    B, H, T, d = q.shape
    dv = bufs["v"].shape[-1]
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    s_out = torch.empty((B, H, dv, d), dtype=torch.float32, device=q.device)
    # the library's scratch (memory entering each chunk), allocated once per input set
    ws_bytes = api.workspace_size(kind, B, H, T, d, dv, chunk, q.dtype)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if kind == "retention":
        return lambda: api.la_chunk_fwd(q, bufs["k"], bufs["v"], bufs["log_gamma"], chunk=chunk, o=o, s_out=s_out,
                                        workspace=ws)
    if kind == "gla":
        return lambda: api.gla_chunk_fwd(q, bufs["k"], bufs["v"], bufs["log_alpha"], chunk=chunk, o=o, s_out=s_out,
                                         workspace=ws)
    if kind == "mamba2":
        return lambda: api.mamba2_chunk_fwd(q, bufs["k"], bufs["v"], bufs["log_alpha"], chunk=chunk, o=o,
                                            s_out=s_out, workspace=ws)
    return lambda: api.gdelta_chunk_fwd(q, bufs["k"], bufs["v"], bufs["log_alpha"], bufs["beta"], chunk=chunk,
                                        o=o, s_out=s_out, workspace=ws)


def time_calls(calls, steps, warmup, torch, graph=False):
    """Run ``warmup`` untimed steps, then ``steps`` timed ones rotating over ``calls``.

    Returns (wall ms per step over the bracketed region, mean kernel ms from HIP events
    recorded on the launching stream). With ``graph`` the timed steps are captured once in
    a HIP graph and replayed: the host then cannot pace a kernel shorter than its own
    launch path, and the per-step time is the region's over the replay. The replay's
    outputs are checked against one eager call per input set first (bit for bit: the
    kernels are deterministic)."""
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    if graph:
        eager = [tuple(t.clone() for t in c() if t is not None) for c in calls]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            outs = [calls[i % len(calls)]() for i in range(steps)]
        g.replay()
        torch.cuda.synchronize()
        for i in range(min(steps, len(calls))):
            got = tuple(t for t in outs[i] if t is not None)
            if not all(torch.equal(a, b) for a, b in zip(got, eager[i])):
                raise RuntimeError("graph replay differs from the eager call")
        region0 = torch.cuda.Event(enable_timing=True)
        region1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        region0.record()
        g.replay()
        region1.record()
        torch.cuda.synchronize()
        ms = region0.elapsed_time(region1) / steps
        return ms, ms
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    region0.record()
    for i in range(steps):
        starts[i].record()
        calls[i % len(calls)]()
        ends[i].record()
    region1.record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return region0.elapsed_time(region1) / steps, float(np.mean(per))


def bench_chunk(name, steps, warmup, torch, api, synthetic, dev, n_sets=N_SETS):
    c = synthetic.CONFIGS[name]
    sets = []
    for s in range(n_sets):
        w = synthetic.config_inputs(name) if s == 0 else None
        if s > 0:
            # further sets: the same recipe with the next seeds (same shapes and distributions)
            base = dict(c)
            kind = base.pop("kind")
            seed = base.pop("seed") + 1000 * s
            fn = {"retention": synthetic.retention_inputs, "gla": synthetic.gla_inputs,
                  "gdelta": synthetic.gdelta_inputs, "mamba2": synthetic.mamba2_inputs}[kind]
            kw = dict(chunk=base["chunk"], dtype=base["dtype"], seed=seed)
            w = fn(base["B"], base["H"], base["T"], base["dk"], base["dv"], **kw)
        sets.append(make_call(c["kind"], api, upload(w, torch, dev), c["chunk"], torch))
        del w
    ms_wall, ms_kernel = time_calls(sets, steps, warmup, torch, graph=True)
    flops, bytes_ = algorithmic_counts(c["kind"], c["B"], c["H"], c["T"], c["dk"], c["chunk"])
    tokens = c["B"] * c["H"] * c["T"]
    return dict(
        workload=name, ms_per_step=ms_wall, kernel_ms=ms_kernel, tokens_per_s=tokens / (ms_wall * 1e-3),
        alg_gbytes=bytes_ / 1e9, alg_gflop=flops / 1e9,
        hbm_gbs=bytes_ / (ms_kernel * 1e-3) / 1e9, mfma_tflops=flops / (ms_kernel * 1e-3) / 1e12)


def bench_decode(steps_total, torch, api, synthetic, dev):
    """The decode workload: 512 sequences x 32 heads, d = 128, fp32 memory, a fresh bf16 token
    and gate per step; ``steps_total`` consecutive steps timed as one region."""
    c = synthetic.CONFIGS["decode_n512h32_d128"]
    N, H, d = c["N"], c["H"], c["dk"]
    w = synthetic.decode_inputs(N, H, d, d, steps=0, seed=c["seed"])
    s = torch.from_numpy(w.s0).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(c["seed"])
    scale = 1.0 / np.sqrt(d)
    q = (torch.randn((steps_total, N, H, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    k = (torch.randn((steps_total, N, H, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    v = (torch.randn((steps_total, N, H, d), generator=gen, device=dev) * scale).to(torch.bfloat16)
    a = torch.sigmoid(torch.randn((steps_total, N, H, d), generator=gen, device=dev) + 2.0)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    for i in range(3):
        api.la_recurrent_step(q[i], k[i], v[i], a[i], s, o=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps_total):
        api.la_recurrent_step(q[i], k[i], v[i], a[i], s, o=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps_total
    bytes_step = N * H * (2 * d * d * 4 + 3 * d * 2 + d * 4 + d * 2)
    return dict(workload="decode_n512h32_d128", steps=steps_total, us_per_step=ms * 1e3,
                hbm_gbs=bytes_step / (ms * 1e-3) / 1e9, hbm_frac=bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                alg_bytes_per_step=bytes_step)


def bench_gdelta_decode(steps_total, torch, api, synthetic, dev):
    """Gated-delta decode at the decode workload's shape (512 sequences x 32 heads, d = 128,
    fp32 memory): a fresh bf16 token per step with the gated-delta workload's recipe
    (q, k = L2(SiLU(N(0,1))), v ~ N(0,1), beta = sigmoid(N(0,1)), alpha = exp(-softplus(N(0,1))/8)
    per sequence and head), drawn on the device; ``steps_total`` steps timed as one region."""
    N, H, d = 512, 32, 128
    w = synthetic.gdelta_decode_inputs(N, H, d, d, steps=0, seed=7)
    s = torch.from_numpy(w.s0).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)

    def unit_silu(x):
        y = x * torch.sigmoid(x)
        return y / y.norm(dim=-1, keepdim=True)

    q = unit_silu(torch.randn((steps_total, N, H, d), generator=gen, device=dev)).to(torch.bfloat16)
    k = unit_silu(torch.randn((steps_total, N, H, d), generator=gen, device=dev)).to(torch.bfloat16)
    v = torch.randn((steps_total, N, H, d), generator=gen, device=dev).to(torch.bfloat16)
    b = torch.sigmoid(torch.randn((steps_total, N, H), generator=gen, device=dev))
    a = torch.exp(-torch.nn.functional.softplus(torch.randn((steps_total, N, H), generator=gen, device=dev)) / 8.0)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    for i in range(3):
        api.gdelta_recurrent_step(q[i], k[i], v[i], a[i], b[i], s, o=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps_total):
        api.gdelta_recurrent_step(q[i], k[i], v[i], a[i], b[i], s, o=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps_total
    bytes_step = N * H * (2 * d * d * 4 + 3 * d * 2 + 2 * 4 + d * 2)
    return dict(workload="gdelta_decode_n512h32_d128", steps=steps_total, us_per_step=ms * 1e3,
                hbm_gbs=bytes_step / (ms * 1e-3) / 1e9, hbm_frac=bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                alg_bytes_per_step=bytes_step)


def bench_gdelta_fused(steps, warmup, torch, api, synthetic, dev):
    """The gated-delta workload from the projections before DeltaNet's feature map, with the
    RMS output norm, through gdelta_chunk_fwd_fused; beside it the same computation with the
    map and the norm as separate torch operations around gdelta_chunk_fwd."""
    B, H, T, d = 4, 16, 8192, 128
    w = synthetic.gdelta_inputs(B, H, T, d, d, chunk=64, dtype="bf16", seed=4, raw_qk=True)
    b = upload(w, torch, dev)
    del w
    weight = torch.linspace(0.5, 1.5, d, device=dev)
    ws = torch.empty(api.workspace_size("gdelta_fused", B, H, T, d, d, 64), dtype=torch.uint8, device=dev)
    o = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    F = torch.nn.functional

    def fused():
        api.gdelta_chunk_fwd_fused(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], chunk=64, o_norm_weight=weight,
                                   o=o, s_out=s_out, workspace=ws)

    def unfused():
        qn = F.normalize(F.silu(b["q"].float()), dim=-1).to(torch.bfloat16)
        kn = F.normalize(F.silu(b["k"].float()), dim=-1).to(torch.bfloat16)
        api.gdelta_chunk_fwd(qn, kn, b["v"], b["log_alpha"], b["beta"], chunk=64, o=o, s_out=s_out, workspace=ws)
        of = o.float()
        return (of * torch.rsqrt(of.pow(2).mean(-1, keepdim=True) + 1e-6) * weight).to(torch.bfloat16)

    ms_f = time_calls([fused], steps, warmup, torch)[1]
    ms_u = time_calls([unfused], steps, warmup, torch)[1]
    return dict(workload="gdelta_fused_b4h16_t8192_d128", kernel_ms=ms_f, unfused_torch_ms=ms_u,
                tokens_per_s=B * H * T / (ms_f * 1e-3), speedup_vs_unfused=ms_u / ms_f)


FP32_VALU_PEAK_TFLOPS = 157.3   # MI355X fp32 vector


def bench_vla(steps, warmup, torch, api, synthetic, dev):
    """Variational linear attention over B8 H16 T4096 d128 (bf16 tokens, fp32 arithmetic), the
    page's ELU+1 ratio readout: one vla_fwd call per step. Algorithmic flops per token-head
    6 d_k^2 + 6 d_v d_k (A u, the rank-1 update and A k^; S k^, the write and S phi(q); the
    denominator's O(d_k) is left out), priced against the fp32 vector peak."""
    name = "vla_b8h16_t4096_d128"
    c = synthetic.CONFIGS[name]
    B, H, T, dk, dv = c["B"], c["H"], c["T"], c["dk"], c["dv"]
    w = synthetic.config_inputs(name)
    b = upload(w, torch, dev)
    uu = torch.from_numpy(w.u).to(dev).to(torch.bfloat16).contiguous()
    del w
    o = torch.empty((B, H, T, dv), dtype=torch.bfloat16, device=dev)
    s_out = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    a_out = torch.empty((B, H, dk, dk), dtype=torch.float32, device=dev)
    n_out = torch.empty((B, H, dk), dtype=torch.float32, device=dev)

    def call():
        api.vla_fwd(b["q"], b["k"], b["v"], uu, lambda0=1.0, o=o, s_out=s_out, a_out=a_out, n_out=n_out)

    ms = time_calls([call], steps, warmup, torch)[1]
    th = B * H * T
    flops = th * (6 * dk * dk + 6 * dv * dk)
    return dict(workload=name, kernel_ms=ms, tokens_per_s=th / (ms * 1e-3), alg_gflop=flops / 1e9,
                fp32_tflops=flops / (ms * 1e-3) / 1e12,
                fp32_valu_frac=flops / (ms * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS,
                heads=B * H, note="two workgroups per (sequence, head), each with half of the memory's rows")


def bench_vla_decode(steps_total, torch, api, synthetic, dev):
    """VLA decode at the decode workload's shape (512 sequences x 32 heads, d = 128), ratio
    readout: the fp32 memory, inverse penalty and denominator vector updated in place, a fresh
    bf16 token per step drawn on the device (q, k, v ~ N(0,1), u ~ N(0,1)/sqrt(d));
    ``steps_total`` steps timed as one region."""
    N, H, d = 512, 32, 128
    w = synthetic.vla_decode_inputs(N, H, d, d, steps=0, seed=9)
    s = torch.from_numpy(w.s0).to(dev)
    a = torch.from_numpy(w.a0).to(dev)
    nd = torch.from_numpy(w.n0).to(dev)
    del w
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    sc = 1.0 / np.sqrt(d)
    q = torch.randn((steps_total, N, H, d), generator=gen, device=dev).to(torch.bfloat16)
    k = torch.randn((steps_total, N, H, d), generator=gen, device=dev).to(torch.bfloat16)
    u = (torch.randn((steps_total, N, H, d), generator=gen, device=dev) * sc).to(torch.bfloat16)
    v = torch.randn((steps_total, N, H, d), generator=gen, device=dev).to(torch.bfloat16)
    o = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
    for i in range(3):
        api.vla_recurrent_step(q[i], k[i], v[i], u[i], s, a, n=nd, o=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps_total):
        api.vla_recurrent_step(q[i], k[i], v[i], u[i], s, a, n=nd, o=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps_total
    # memory, penalty and denominator read and written; q, k, u, v read; o written
    bytes_step = N * H * (2 * (d * d + d * d + d) * 4 + 4 * d * 2 + d * 2)
    return dict(workload="vla_decode_n512h32_d128", steps=steps_total, us_per_step=ms * 1e3,
                hbm_gbs=bytes_step / (ms * 1e-3) / 1e9, hbm_frac=bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                alg_bytes_per_step=bytes_step)


def bench_backward(name, steps, warmup, torch, api, synthetic, dev):
    """Backward of a retention, scalar-decay or GLA workload (forward state pass, reverse state
    pass, gradient pass, and for the first two a gate pass) with a seeded dO and ds_out; beside it
    the forward of the same workload. Algorithmic flops per token-head 8Cd + 10d^2 (the two
    state passes 2d^2 each; Q K^T, dO V^T, dO^T A1, Q^T A2, K^T A2^T 2Cd each over the
    C x C block; R K^T, R^T V^T, S_in^T dO^T 2d^2 each); bytes: read q, k, v, dO, write dq,
    dk, dv (7 d bf16 per token-head), the gates (GLA: read and their gradient written, 8 d
    bytes) and three d x d fp32 memories per head."""
    c = synthetic.CONFIGS[name]
    B, H, T, d, C = c["B"], c["H"], c["T"], c["dk"], c["chunk"]
    w = synthetic.config_inputs(name)
    b = upload(w, torch, dev)
    del w
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    dout = (torch.randn((B, H, T, d), generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
    ds_out = torch.randn((B, H, d, d), generator=g, device=dev) * 0.1
    ws = torch.empty(api.bwd_workspace_size(B, H, T, d, d, C), dtype=torch.uint8, device=dev)
    if c["kind"] == "retention":
        bwd = lambda: api.la_chunk_bwd(b["q"], b["k"], b["v"], b["log_gamma"], dout, ds_out=ds_out, chunk=C,
                                       workspace=ws)
        gate_bytes = 0
    elif c["kind"] == "gla":
        ws = torch.empty(api.bwd_workspace_size(B, H, T, d, d, C, gla=True), dtype=torch.uint8, device=dev)
        bwd = lambda: api.gla_chunk_bwd(b["q"], b["k"], b["v"], b["log_alpha"], dout, ds_out=ds_out, chunk=C,
                                        workspace=ws)
        gate_bytes = 8 * d
    else:
        bwd = lambda: api.mamba2_chunk_bwd(b["q"], b["k"], b["v"], b["log_alpha"], dout, ds_out=ds_out, chunk=C,
                                           workspace=ws)
        gate_bytes = 8
    fwd = make_call(c["kind"], api, b, C, torch)
    ms_b = time_calls([bwd], steps, warmup, torch)[1]
    ms_f = time_calls([fwd], steps, warmup, torch)[1]
    th = B * H * T
    flops = th * (8 * C * d + 10 * d * d)
    bytes_ = th * (7 * d * 2 + gate_bytes) + 3 * B * H * d * d * 4
    return dict(workload=name + "_bwd", kernel_ms=ms_b, fwd_kernel_ms=ms_f, bwd_over_fwd=ms_b / ms_f,
                tokens_per_s=th / (ms_b * 1e-3), alg_gflop=flops / 1e9, alg_gbytes=bytes_ / 1e9,
                mfma_frac=flops / (ms_b * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                hbm_frac=bytes_ / (ms_b * 1e-3) / 1e9 / HBM_PEAK_GBS)


KERNEL_SOURCES = ("gated_linear_recurrences_amd/csrc/chunk_fused.hpp",
                  "gated_linear_recurrences_amd/csrc/chunk_state.hpp",
                  "gated_linear_recurrences_amd/csrc/chunk_output.hpp",
                  "gated_linear_recurrences_amd/csrc/chunk_two_pass.hpp",
                  "gated_linear_recurrences_amd/csrc/chunk_common.hpp",
                  "gated_linear_recurrences_amd/csrc/chunk_bf16_retention_c64.hip",
                  "gated_linear_recurrences_amd/csrc/device_common.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the timed kernel from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size), or None when the
    kernel sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash() or rec.get("workload") != MAIN:
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_CAL_MB = 512   # size of the plain copy the counter runs are scaled by
# kernel of one retention call (bf16, chunk 64, d_k = d_v = 128, 16-channel value slices,
# fixed gate), as rocprofv3 names it
TRAFFIC_KERNELS = ("glr::ck::fused_kernel<64, 128, 128, 1, 0>",)


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, match):
    """{dispatch id: summed counter value} over the dispatches whose kernel name matches."""
    out = {}
    for r in rows:
        if match(r["Kernel_Name"]):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


def summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """HBM bytes per retention call from FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch),
    each scaled by what the same counter reads for a plain copy of known size; writes
    profiles/pmc_traffic.json and prints the table of the profile summary."""
    is_copy = lambda k: "copy" in k.lower()
    res = {}
    for label, d, cd in (("fetch", fetch_dir, copy_fetch_dir), ("write", write_dir, copy_write_dir)):
        rows = _counter_rows(d)
        per_kernel = {}
        for t in TRAFFIC_KERNELS:
            disp = _per_dispatch(rows, lambda k, t=t: t in k)
            per_kernel[t] = (sum(disp.values()) / len(disp), len(disp))
        copy = _per_dispatch(_counter_rows(cd), is_copy)
        copy_kib = max(copy.values())     # the 512 MB copy, not small incidental copies
        res[label] = (per_kernel, copy_kib)
    copy_bytes = int(COPY_CAL_MB * 1e6) // 4 * 4   # the copy of --copy-calibration COPY_CAL_MB
    rec = {"workload": MAIN, "kernels": list(TRAFFIC_KERNELS), "source_sha256": kernel_source_hash(),
           "copy_calibration_bytes": copy_bytes}
    total = 0.0
    lines = ["| quantity | raw counter (KiB / dispatch) | scale | bytes / call |", "|---|---|---|---|"]
    for label in ("fetch", "write"):
        per_kernel, copy_kib = res[label]
        scale = copy_bytes / 1024.0 / copy_kib
        lines.append(f"| plain copy of {copy_bytes:,} B, {label.upper()}_SIZE | {copy_kib:.0f} | "
                     f"{copy_bytes / 1024:.0f} / raw = {scale:.4f} | {copy_bytes:,} |")
        part = 0.0
        for t, (kib, n) in per_kernel.items():
            b = kib * 1024.0 * scale
            part += b
            lines.append(f"| `{t}...` {label.upper()}_SIZE ({n} dispatches) | {kib:.0f} | {scale:.4f} | {b:,.0f} |")
        rec[f"{label}_scale"] = scale
        rec[f"{label}_bytes_per_call"] = part
        total += part
    rec["hbm_bytes_per_launch"] = total
    lines.append(f"| **total HBM traffic per call** | | | **{total:,.0f}** |")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


def kernel_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Per-kernel HBM bytes per dispatch for every library kernel in a FETCH_SIZE and a
    WRITE_SIZE run, each scaled by the same counter on the plain copy; prints a table."""
    is_copy = lambda k: "copy" in k.lower()
    copy_bytes = int(COPY_CAL_MB * 1e6) // 4 * 4
    cols = {}
    for label, d, cd in (("fetch", fetch_dir, copy_fetch_dir), ("write", write_dir, copy_write_dir)):
        rows = _counter_rows(d)
        scale = copy_bytes / 1024.0 / max(_per_dispatch(_counter_rows(cd), is_copy).values())
        names = sorted({r["Kernel_Name"] for r in rows if "glr::" in r["Kernel_Name"]})
        for name in names:
            disp = _per_dispatch(rows, lambda k, name=name: k == name)
            cols.setdefault(name, {})[label] = (sum(disp.values()) / len(disp) * 1024.0 * scale, len(disp))
        cols.setdefault("_scale", {})[label] = scale
    lines = [f"FETCH_SIZE scale {cols['_scale']['fetch']:.4f}, WRITE_SIZE scale {cols['_scale']['write']:.4f} "
             f"(plain copy of {copy_bytes:,} B)", "",
             "| kernel | dispatches | read bytes / dispatch | written bytes / dispatch |", "|---|---|---|---|"]
    for name, c in cols.items():
        if name == "_scale":
            continue
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        f, nf = c.get("fetch", (float("nan"), 0))
        w, _ = c.get("write", (float("nan"), 0))
        lines.append(f"| `{short}` | {nf} | {f:,.0f} | {w:,.0f} |")
    print("\n".join(lines))


def trace_table(trace_dir):
    """Average, min and max duration per library kernel and grid size from a rocprofv3
    --kernel-trace run (the *_kernel_trace.csv under trace_dir); prints a table."""
    import csv
    import glob
    import re
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    agg = {}
    for r in rows:
        name = r["Kernel_Name"]
        if "glr::" not in name:
            continue
        name = name.replace("void ", "").replace("(anonymous namespace)::", "")
        name = re.sub(r"\(.*$", "", name.replace("glr::ck::", "").replace("glr::", ""))
        key = (name, r.get("Grid_Size_X") or r.get("Grid_Size", ""))
        agg.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | grid (threads) | calls | average (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|---|")
    for (name, grid), d in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name}` | {grid} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")


def copy_calibration(mbytes, steps, torch):
    """A plain device copy of ``mbytes`` MB, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = int(mbytes * 1e6) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "steps": steps}))


def cpu_baseline(synthetic, budget_s=12.0):
    """The fp64 oracle (chunkwise form) on the host: whole retention batches of the timed
    workload, repeated until ``budget_s`` has elapsed. numpy's einsum runs on one thread."""
    import oracle
    w = synthetic.config_inputs(MAIN)
    c = synthetic.CONFIGS[MAIN]
    t0 = time.perf_counter()
    done = 0
    while True:
        for b in range(c["B"]):
            oracle.retention_chunkwise(w.q[b:b + 1], w.k[b:b + 1], w.v[b:b + 1], w.log_gamma, c["chunk"])
            done += c["H"] * c["T"]
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"fp64 chunkwise retention oracle on {done // (c['H'] * c['T'])} batch rows of "
                      f"{MAIN} (H={c['H']}, T={c['T']}, d=128) in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-others", action="store_true",
                    help="skip the GLA, gated-delta, scalar-decay and decode workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="only run a plain device copy of MB megabytes --steps times (counter scaling)")
    ap.add_argument("--kernel-traffic", nargs=4, metavar="DIR",
                    help="per-kernel HBM bytes from FETCH/WRITE runs and the copy calibration runs")
    ap.add_argument("--trace-table", metavar="DIR",
                    help="print per-kernel durations from a rocprofv3 --kernel-trace output folder")
    ap.add_argument("--summarize-traffic", nargs=4, metavar="DIR",
                    help="FETCH_SIZE and WRITE_SIZE counter dirs of a bench run, then of a copy run: "
                         "write profiles/pmc_traffic.json")
    args = ap.parse_args()
    if args.trace_table:
        trace_table(args.trace_table)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.kernel_traffic:
        kernel_traffic(*args.kernel_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the recurrences shard over (batch, head) with no "
              "communication, so only --gpus 1 is run here", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_linear_recurrences_amd import api, synthetic
    dev = "cuda"
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, args.steps, torch)
        return

    main_r = bench_chunk(MAIN, args.steps, args.warmup, torch, api, synthetic, dev)
    others = {}
    if not args.no_others:
        for name in ("gla_b8h16_t4096_d128", "gdelta_b4h16_t8192_d128", "mamba2_b8h16_t4096_d128"):
            r = bench_chunk(name, max(20, args.steps // 4), max(3, args.warmup // 4), torch, api, synthetic, dev,
                            n_sets=1)
            r["hbm_frac"] = r["hbm_gbs"] / HBM_PEAK_GBS
            r["mfma_frac"] = r["mfma_tflops"] / MFMA_BF16_PEAK_TFLOPS
            others[name] = r
            torch.cuda.empty_cache()
        others["decode_n512h32_d128"] = bench_decode(args.decode_steps, torch, api, synthetic, dev)
        torch.cuda.empty_cache()
        others["gdelta_fused_b4h16_t8192_d128"] = bench_gdelta_fused(max(20, args.steps // 4),
                                                                     max(3, args.warmup // 4), torch, api,
                                                                     synthetic, dev)
        torch.cuda.empty_cache()
        others["gdelta_decode_n512h32_d128"] = bench_gdelta_decode(min(args.decode_steps, 200), torch, api,
                                                                   synthetic, dev)
        torch.cuda.empty_cache()
        for name in (MAIN, "mamba2_b8h16_t4096_d128", "gla_b8h16_t4096_d128"):
            others[name + "_bwd"] = bench_backward(name, max(20, args.steps // 4), max(3, args.warmup // 4), torch,
                                                   api, synthetic, dev)
            torch.cuda.empty_cache()
        others["vla_b8h16_t4096_d128"] = bench_vla(max(5, args.steps // 40), 1, torch, api, synthetic, dev)
        torch.cuda.empty_cache()
        others["vla_decode_n512h32_d128"] = bench_vla_decode(min(args.decode_steps, 50), torch, api, synthetic, dev)
        torch.cuda.empty_cache()

    cfg = synthetic.CONFIGS[MAIN]
    out = {
        "metric": "chunked fwd tokens/s (B·H·T/s) + % bf16 MFMA peak; decode step HBM GB/s",
        "value": main_r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": MAIN, "B": cfg["B"], "H": cfg["H"], "T": cfg["T"], "d_k": cfg["dk"],
                   "d_v": cfg["dv"], "chunk": cfg["chunk"], "decay": "1 - 2^(-5-h)", "state": "fp32",
                   "input_sets_rotated": N_SETS},
        "roofline": {"bound": "hbm", "achieved": main_r["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": main_r["hbm_gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel_ms": main_r["kernel_ms"], "alg_bytes_per_launch": main_r["alg_gbytes"] * 1e9,
                     "kernels": "single-pass forward (one call)"},
        "mfma": {"achieved": main_r["mfma_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": main_r["mfma_tflops"] / MFMA_BF16_PEAK_TFLOPS,
                 "alg_flop_per_launch": main_r["alg_gflop"] * 1e9},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(synthetic)
    if others:
        out["others"] = others
    print(json.dumps(out))


if __name__ == "__main__":
    main()
