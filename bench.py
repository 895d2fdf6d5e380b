#!/usr/bin/env python3
"""Throughput of the chunked forwards on one MI355X, with their rooflines and the CPU oracle beside them.

A step is one call of the gated delta rule's chunked forward - every stage of the hot
path (the cumulative gates and the per-chunk UT factor T_U in a chunk-parallel prep; the
memory carried from chunk to chunk, the pseudo-values U, the decayed triangle, P U, the
memory readout and the stores in one single-pass kernel) - over one batch of the gated
delta rule workload: B=4, H=16, T=8192, d_k=d_v=128, bf16 q/k = L2(SiLU(N(0,1))), v ~
N(0,1), beta = sigmoid(N(0,1)), log alpha = -softplus(N(0,1))/8, chunk 64, fp32 memory:
the largest single-GPU configuration, and the only one whose MFMA ceiling (51%) admits the
40% target. Inputs are resident in HBM before timing; two input sets are rotated.

Printed: one JSON line. ``value`` is tokens/s (B*H*T per second); ``roofline`` prices the
call (both kernels, timed with HIP events on the launching stream around one HIP-graph
replay of the timed steps, so that host launches do not pace it) against HBM with the
algorithmic bytes of the method (q, k, v and the gates read, o and the final memory
written); ``traffic`` is the HBM traffic the counters measured for one call; ``mfma``
gives the same call against the dense bf16 MFMA peak, with the flops counted over the
causal tiles of each chunk (and the hardware's own MFMA counters when recorded);
``cpu_baseline`` times the fp64 oracle on the host's cores; ``others`` reports the other
chunked workloads (retention B4 H8 T2048, GLA and the scalar data-dependent decay at B8
H16 T4096) each with its own roofline, decode (per-channel gate, gated delta rule), the
gated delta rule with its feature map and output norm fused in, GLA with its output
LayerNorm fused in (each beside the unfused torch form), the backward of
retention, the scalar decay, GLA and the gated delta rule (beside their forward), and variational linear
attention (whole sequences, and decode).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-others] [--no-cpu]
    python bench.py --counter-run                       (each chunked workload, three calls, for rocprofv3 --pmc)
    python bench.py --copy-calibration MB --steps K      (plain copy, for counter scaling)
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
    python bench.py --summarize-mfma MFMA_DIR
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
N_CU = 256

MAIN = "gdelta_b4h16_t8192_d128"
# the chunked workloads, each priced against its own roofline; rotated input sets (enough to
# exceed the 256 MB Infinity Cache: the retention batch is 67 MB per set)
CHUNKED = ("gdelta_b4h16_t8192_d128", "retention_b4h8_t2048_d128", "gla_b8h16_t4096_d128", "mamba2_b8h16_t4096_d128")
N_SETS = {"gdelta_b4h16_t8192_d128": 2, "retention_b4h8_t2048_d128": 5, "gla_b8h16_t4096_d128": 1,
          "mamba2_b8h16_t4096_d128": 1}
# library kernels of one call of each chunked workload (d_k = d_v = 128, chunk 64), as rocprofv3 names them
WORKLOAD_KERNELS = {
    "gdelta_b4h16_t8192_d128": ("glr::ck::delta_tfac_kernel<64, 128>",
                                "glr::ck::delta_sp_kernel<64, 128, 128, 32, 3, 1, false, false>"),
    "retention_b4h8_t2048_d128": ("glr::ck::delta_sp_kernel<64, 128, 128, 16, 0, 1, false, false>",),
    "gla_b8h16_t4096_d128": ("glr::ck::gla_sp_kernel<128, 128, 64>",),
    "mamba2_b8h16_t4096_d128": ("glr::ck::delta_sp_kernel<64, 128, 128, 64, 2, 2, false, false>",),
}


def algorithmic_counts(kind, B, H, T, d, chunk, elem_bytes=2):
    """Algorithmic flops and HBM bytes of one chunked-forward call.

    Bytes: read q, k, v (and the gates), write o and the final memory.
    Flops per token-head (chunk C, head size d), counted over the causal tiles (j <= i) of
    each C x C block, which is all the method needs: retention, the scalar decay and GLA
    2d(C + 1) + 4d^2 (q.k^T and P.V over the lower triangle, S q and k^T v); the gated delta
    rule 4Cd + 2d + 6d^2 + 2C^2/3 (K K^T strictly lower, Q K^T, T_U R and P U over the lower
    triangle; K S^T, Q S^T and the carry K^T U; the triangular solve)."""
    th = B * H * T
    tok_bytes = 4 * d * elem_bytes
    gate_bytes = {"retention": 0, "mamba2": 4, "gla": 4 * d, "gdelta": 8}[kind]
    state_bytes = B * H * d * d * 4
    bytes_ = th * (tok_bytes + gate_bytes) + state_bytes
    if kind == "gdelta":
        flops = th * (4 * chunk * d + 2 * d + 6 * d * d + 2 * chunk * chunk / 3)
    else:
        flops = th * (2 * d * (chunk + 1) + 4 * d * d)
    return flops, bytes_


def full_block_flops(kind, B, H, T, d, chunk):
    """The same products counted over the whole C x C block (the survey's count): 4Cd + 4d^2,
    or 8Cd + 6d^2 + 2C^2/3 for the gated delta rule; reported beside the causal count."""
    th = B * H * T
    if kind == "gdelta":
        return th * (8 * chunk * d + 6 * d * d + 2 * chunk * chunk / 3)
    return th * (4 * chunk * d + 4 * d * d)


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


def bench_chunk(name, steps, warmup, torch, api, synthetic, dev, n_sets=None):
    c = synthetic.CONFIGS[name]
    n_sets = N_SETS.get(name, 1) if n_sets is None else n_sets
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
        input_sets_rotated=n_sets, alg_gbytes=bytes_ / 1e9, alg_gflop=flops / 1e9,
        hbm_gbs=bytes_ / (ms_kernel * 1e-3) / 1e9, mfma_tflops=flops / (ms_kernel * 1e-3) / 1e12)


def roofline_block(name, r, synthetic):
    """The call priced against HBM (the bound of every chunked workload: their intensities,
    64 - 161 flop/byte, lie below the ridge of ~315) and against the dense bf16 MFMA peak."""
    c = synthetic.CONFIGS[name]
    flops, bytes_ = algorithmic_counts(c["kind"], c["B"], c["H"], c["T"], c["dk"], c["chunk"])
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    ai = flops / bytes_
    roof = {"bound": "hbm", "achieved": r["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": r["hbm_gbs"] / HBM_PEAK_GBS, "traffic": measured_traffic(name),
            "kernel_ms": r["kernel_ms"], "alg_bytes_per_launch": bytes_,
            "kernels": " + ".join(k.split("::")[-1] for k in WORKLOAD_KERNELS[name]) + " (one call)"}
    mf = {"achieved": r["mfma_tflops"], "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
          "frac": r["mfma_tflops"] / MFMA_BF16_PEAK_TFLOPS, "alg_flop_per_launch": flops,
          "flop_count": "causal tiles", "ceiling_frac": min(1.0, ai / ridge),
          "frac_full_block_count": full_block_flops(c["kind"], c["B"], c["H"], c["T"], c["dk"], c["chunk"])
          / (r["kernel_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    hw = measured_mfma(name)
    if hw is not None:
        mf["counters"] = dict(hw, hw_tflops=hw["mfma_flop_per_call"] / (r["kernel_ms"] * 1e-3) / 1e12)
    return roof, mf


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


def time_pair(fused, unfused, steps, warmup, torch):
    """Kernel ms of a fused call and of its unfused form: both warmed first (whichever is timed
    first would otherwise also pay for the clocks ramping up), then each timed."""
    time_calls([fused, unfused], 2 * warmup, 2 * warmup, torch)
    return time_calls([fused], steps, warmup, torch)[1], time_calls([unfused], steps, warmup, torch)[1]


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

    ms_f, ms_u = time_pair(fused, unfused, steps, warmup, torch)
    return dict(workload="gdelta_fused_b4h16_t8192_d128", kernel_ms=ms_f, unfused_torch_ms=ms_u,
                tokens_per_s=B * H * T / (ms_f * 1e-3), speedup_vs_unfused=ms_u / ms_f)


def bench_gla_layernorm(steps, warmup, torch, api, synthetic, dev):
    """The GLA workload (B8 H16 T4096 d128) with its output LayerNorm (gla_chunk_fwd_fused: the
    single pass, then the library's layer norm over the output rows); beside it gla_chunk_fwd
    followed by torch's layer_norm on o."""
    name = "gla_b8h16_t4096_d128"
    c = synthetic.CONFIGS[name]
    B, H, T, d = c["B"], c["H"], c["T"], c["dk"]
    b = upload(synthetic.config_inputs(name), torch, dev)
    weight = torch.linspace(0.5, 1.5, d, device=dev)
    bias = torch.linspace(-0.2, 0.2, d, device=dev)
    ws = torch.empty(max(api.workspace_size("gla", B, H, T, d, d, 64), 16), dtype=torch.uint8, device=dev)
    o = torch.empty((B, H, T, d), dtype=torch.bfloat16, device=dev)
    s_out = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    F = torch.nn.functional

    def fused():
        api.gla_chunk_fwd_fused(b["q"], b["k"], b["v"], b["log_alpha"], weight, o_norm_bias=bias, o_norm_eps=1e-5,
                                chunk=64, o=o, s_out=s_out, workspace=ws)

    def unfused():
        api.gla_chunk_fwd(b["q"], b["k"], b["v"], b["log_alpha"], chunk=64, o=o, s_out=s_out, workspace=ws)
        return F.layer_norm(o.float(), (d,), weight, bias, 1e-5).to(torch.bfloat16)

    ms_f, ms_u = time_pair(fused, unfused, steps, warmup, torch)
    return dict(workload="gla_layernorm_b8h16_t4096_d128", kernel_ms=ms_f, unfused_torch_ms=ms_u,
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
    """Backward of a retention, scalar-decay, GLA or gated-delta workload (forward state pass,
    reverse state pass, gradient pass, and for the first two a gate pass; for the gated delta rule
    also the chunk prep and maps) with a seeded dO and ds_out; beside it the forward of the same
    workload. The flop count below is the decay variants'; for the gated delta rule it is a
    lower bound. Algorithmic flops per token-head 8Cd + 10d^2 (the two
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
    if c["kind"] == "gdelta":
        ws = torch.empty(api.bwd_workspace_size(B, H, T, d, d, C, gdelta=True), dtype=torch.uint8, device=dev)
        bwd = lambda: api.gdelta_chunk_bwd(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], dout, ds_out=ds_out,
                                           chunk=C, workspace=ws)
        gate_bytes = 16
    elif c["kind"] == "retention":
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


CSRC = os.path.join(ROOT, "gated_linear_recurrences_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "pmc_mfma.json")


def kernel_source_hash():
    """SHA-256 over every kernel source of the library: recorded counters are reported only
    while the sources they were measured on are unchanged."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hpp", ".hip", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()


def _recorded(path, name):
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("workloads", {}).get(name)


def measured_traffic(name=MAIN):
    """HBM bytes per call of a chunked workload from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE of its kernels, scaled by a plain copy of known size), or None
    when the kernel sources have changed since the counters were taken."""
    rec = _recorded(TRAFFIC_FILE, name)
    return None if rec is None else rec["hbm_bytes_per_call"]


def measured_mfma(name=MAIN):
    """MFMA counters per call of a chunked workload (rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE of its kernels), or None when stale."""
    return _recorded(MFMA_FILE, name)


COPY_CAL_MB = 512   # size of the plain copy the counter runs are scaled by


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


def _per_dispatch(rows, match, counter=None):
    """{dispatch id: summed counter value} over the dispatches whose kernel name matches."""
    out = {}
    for r in rows:
        if match(r["Kernel_Name"]) and (counter is None or r["Counter_Name"] == counter):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


def _kernel_match(kernel):
    # rocprofv3 names carry "void " and the argument list: match the name up to its arguments
    return lambda k: k.replace("void ", "").split("(")[0].strip() == kernel


def summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """HBM bytes per call of every chunked workload from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch) of ``bench.py --counter-run``, each scaled by what the same counter reads for a
    plain copy of known size; writes profiles/pmc_traffic.json and prints the table of the
    profile summary."""
    is_copy = lambda k: "copy" in k.lower()
    copy_bytes = int(COPY_CAL_MB * 1e6) // 4 * 4   # the copy of --copy-calibration COPY_CAL_MB
    scale = {}
    rows = {}
    for label, d, cd in (("fetch", fetch_dir, copy_fetch_dir), ("write", write_dir, copy_write_dir)):
        rows[label] = _counter_rows(d)
        copy_kib = max(_per_dispatch(_counter_rows(cd), is_copy).values())   # the 512 MB copy
        scale[label] = copy_bytes / 1024.0 / copy_kib
    rec = {"source_sha256": kernel_source_hash(), "copy_calibration_bytes": copy_bytes,
           "fetch_scale": scale["fetch"], "write_scale": scale["write"], "workloads": {}}
    lines = [f"FETCH_SIZE scale {scale['fetch']:.4f}, WRITE_SIZE scale {scale['write']:.4f} "
             f"(plain copy of {copy_bytes:,} B: raw KiB x scale = bytes / 1024)", "",
             "| workload | kernel | dispatches | read bytes / dispatch | written bytes / dispatch |",
             "|---|---|---|---|---|"]
    for name, kernels in WORKLOAD_KERNELS.items():
        w = {"kernels": list(kernels), "fetch_bytes_per_call": 0.0, "write_bytes_per_call": 0.0}
        ok = True
        for kern in kernels:
            per = {}
            for label in ("fetch", "write"):
                disp = _per_dispatch(rows[label], _kernel_match(kern))
                if not disp:
                    ok = False
                    break
                per[label] = (sum(disp.values()) / len(disp) * 1024.0 * scale[label], len(disp))
                w[f"{label}_bytes_per_call"] += per[label][0]
            if not ok:
                break
            lines.append(f"| {name} | `{kern.split('::')[-1]}` | {per['fetch'][1]} | {per['fetch'][0]:,.0f} | "
                         f"{per['write'][0]:,.0f} |")
        if ok:
            w["hbm_bytes_per_call"] = w["fetch_bytes_per_call"] + w["write_bytes_per_call"]
            rec["workloads"][name] = w
            lines.append(f"| **{name}** | **total per call** | | **{w['fetch_bytes_per_call']:,.0f}** | "
                         f"**{w['write_bytes_per_call']:,.0f}** |")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print("\n".join(lines))


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
N_XCD = 8   # GRBM_GUI_ACTIVE comes summed over the XCDs


def summarize_mfma(mfma_dir):
    """MFMA counters per call of every chunked workload from one rocprofv3 --pmc run of
    ``bench.py --counter-run`` (SQ_INSTS_VALU_MFMA_MOPS_BF16: bf16 MFMA work in units of 512
    flops; SQ_VALU_MFMA_BUSY_CYCLES: cycles the MFMA units were busy, summed over the chip;
    GRBM_GUI_ACTIVE: cycles the GPU was busy, which rocprofv3 sums over the 8 XCDs, so it is
    divided by 8). Busy fraction = MFMA busy cycles / (GPU busy cycles x 256 CUs x 4 SIMDs).
    Writes profiles/pmc_mfma.json and prints a table."""
    rows = _counter_rows(mfma_dir)
    rec = {"source_sha256": kernel_source_hash(), "counters": list(MFMA_COUNTERS), "workloads": {}}
    lines = ["| workload | kernel | dispatches | MFMA bf16 flop / dispatch | MFMA busy cycles | GPU busy cycles | "
             "MFMA busy fraction |", "|---|---|---|---|---|---|---|"]
    for name, kernels in WORKLOAD_KERNELS.items():
        tot = {"mops": 0.0, "busy": 0.0, "gui": 0.0}
        ok = True
        for kern in kernels:
            vals = {}
            for key, counter in (("mops", MFMA_COUNTERS[0]), ("busy", MFMA_COUNTERS[1]), ("gui", MFMA_COUNTERS[2])):
                disp = _per_dispatch(rows, _kernel_match(kern), counter)
                if not disp:
                    ok = False
                    break
                vals[key] = sum(disp.values()) / len(disp) / (N_XCD if key == "gui" else 1)
                n = len(disp)
            if not ok:
                break
            for key in tot:
                tot[key] += vals[key]
            frac = vals["busy"] / (vals["gui"] * N_CU * 4) if vals["gui"] else float("nan")
            lines.append(f"| {name} | `{kern.split('::')[-1]}` | {n} | {vals['mops'] * 512:,.0f} | {vals['busy']:,.0f} | "
                         f"{vals['gui']:,.0f} | {frac:.3f} |")
        if ok:
            rec["workloads"][name] = {"kernels": list(kernels), "mfma_flop_per_call": tot["mops"] * 512,
                                      "mfma_busy_cycles_per_call": tot["busy"], "gpu_busy_cycles_per_call": tot["gui"],
                                      "mfma_busy_frac": tot["busy"] / (tot["gui"] * N_CU * 4) if tot["gui"] else None}
    with open(MFMA_FILE, "w") as f:
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


def _oracle_heads(args):
    """One worker of the CPU baseline: the oracle's chunkwise gated delta rule on a block of
    (batch, head) sequences. Runs in a fresh process with one BLAS thread."""
    q, k, v, la, beta, chunk = args
    import oracle
    t0 = time.perf_counter()
    oracle.gdelta_chunkwise(q, k, v, la, beta, chunk)
    return time.perf_counter() - t0


def cpu_baseline(synthetic, cores=None, heads_per_task=1):
    """The fp64 oracle (chunkwise form, as written) on the host's cores: the sequences of the
    timed workload split over ``cores`` worker processes (one BLAS thread each), one sequence
    per task; tokens per second of wall time over the sample."""
    import concurrent.futures
    import multiprocessing as mp
    c = synthetic.CONFIGS[MAIN]
    # the GPU machine gives one GPU's job 16 host cores, whatever os.cpu_count() shows
    cores = cores or max(1, min(16, os.cpu_count() or 1))
    w = synthetic.config_inputs(MAIN)
    B, H, T = c["B"], c["H"], c["T"]
    n_seq = min(B * H, 2 * cores)   # a bounded sample: two sequences per core
    tasks = []
    for i in range(0, n_seq, heads_per_task):
        sl = [(j // H, j % H) for j in range(i, min(i + heads_per_task, n_seq))]
        b = np.array([x[0] for x in sl]); h = np.array([x[1] for x in sl])
        tasks.append((w.q[b, h][None], w.k[b, h][None], w.v[b, h][None], w.log_alpha[b, h][None], w.beta[b, h][None],
                      c["chunk"]))
    del w
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with concurrent.futures.ProcessPoolExecutor(cores, mp_context=ctx) as ex:
            list(ex.map(_oracle_heads, tasks[:cores]))   # start the workers (imports) before timing
            t0 = time.perf_counter()
            list(ex.map(_oracle_heads, tasks))
            el = time.perf_counter() - t0
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    tokens = n_seq * T
    return {"value": tokens / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 chunkwise gated-delta oracle on {n_seq} of the {B * H} sequences of {MAIN} "
                      f"(T={T}, d=128, chunk {c['chunk']}), {cores} worker processes with one BLAS thread each, "
                      f"{el:.1f} s wall"}


def counter_run(torch, api, synthetic, dev, calls=3):
    """Each chunked workload, ``calls`` eager calls and nothing else: the run rocprofv3 --pmc
    takes its per-kernel counters from."""
    for name in CHUNKED:
        c = synthetic.CONFIGS[name]
        call = make_call(c["kind"], api, upload(synthetic.config_inputs(name), torch, dev), c["chunk"], torch)
        for _ in range(calls):
            call()
        torch.cuda.synchronize()
        del call
        torch.cuda.empty_cache()
    print(json.dumps({"counter_run": list(CHUNKED), "calls": calls}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-others", action="store_true",
                    help="only the headline workload (no other chunked workloads, decode, backward or VLA)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--counter-run", action="store_true",
                    help="only run each chunked workload three times (for rocprofv3 --pmc)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB",
                    help="only run a plain device copy of MB megabytes --steps times (counter scaling)")
    ap.add_argument("--kernel-traffic", nargs=4, metavar="DIR",
                    help="per-kernel HBM bytes from FETCH/WRITE runs and the copy calibration runs")
    ap.add_argument("--trace-table", metavar="DIR",
                    help="print per-kernel durations from a rocprofv3 --kernel-trace output folder")
    ap.add_argument("--summarize-traffic", nargs=4, metavar="DIR",
                    help="FETCH_SIZE and WRITE_SIZE counter dirs of a --counter-run, then of a copy run: "
                         "write profiles/pmc_traffic.json")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="MFMA counter dir of a --counter-run: write profiles/pmc_mfma.json")
    args = ap.parse_args()
    if args.trace_table:
        trace_table(args.trace_table)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
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
    if args.counter_run:
        counter_run(torch, api, synthetic, dev)
        return

    main_r = bench_chunk(MAIN, args.steps, args.warmup, torch, api, synthetic, dev)
    print(f"[bench] {MAIN}: {main_r['kernel_ms'] * 1e3:.1f} us per call", file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    others = {}
    if not args.no_others:
        for name in CHUNKED[1:]:
            r = bench_chunk(name, max(20, args.steps // 2), max(3, args.warmup // 2), torch, api, synthetic, dev)
            r["roofline"], r["mfma"] = roofline_block(name, r, synthetic)
            others[name] = r
            print(f"[bench] {name}: {r['kernel_ms'] * 1e3:.1f} us per call", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        others["decode_n512h32_d128"] = bench_decode(args.decode_steps, torch, api, synthetic, dev)
        torch.cuda.empty_cache()
        others["gdelta_fused_b4h16_t8192_d128"] = bench_gdelta_fused(max(20, args.steps // 4),
                                                                     max(3, args.warmup // 4), torch, api,
                                                                     synthetic, dev)
        torch.cuda.empty_cache()
        others["gla_layernorm_b8h16_t4096_d128"] = bench_gla_layernorm(max(20, args.steps // 4),
                                                                       max(3, args.warmup // 4), torch, api,
                                                                       synthetic, dev)
        torch.cuda.empty_cache()
        others["gdelta_decode_n512h32_d128"] = bench_gdelta_decode(min(args.decode_steps, 200), torch, api,
                                                                   synthetic, dev)
        torch.cuda.empty_cache()
        for name in ("retention_b4h8_t2048_d128", "mamba2_b8h16_t4096_d128", "gla_b8h16_t4096_d128",
                     "gdelta_b4h16_t8192_d128"):
            others[name + "_bwd"] = bench_backward(name, max(20, args.steps // 4), max(3, args.warmup // 4), torch,
                                                   api, synthetic, dev)
            torch.cuda.empty_cache()
        others["vla_b8h16_t4096_d128"] = bench_vla(max(5, args.steps // 20), 1, torch, api, synthetic, dev)
        torch.cuda.empty_cache()
        others["vla_decode_n512h32_d128"] = bench_vla_decode(min(args.decode_steps, 50), torch, api, synthetic, dev)
        torch.cuda.empty_cache()
        print("[bench] other workloads done", file=sys.stderr, flush=True)

    cfg = synthetic.CONFIGS[MAIN]
    roof, mf = roofline_block(MAIN, main_r, synthetic)
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
                   "d_v": cfg["dv"], "chunk": cfg["chunk"], "keys": "L2(SiLU(N(0,1)))",
                   "gates": "log alpha = -softplus(N(0,1))/8, beta = sigmoid(N(0,1))", "state": "fp32",
                   "input_sets_rotated": main_r["input_sets_rotated"]},
        "roofline": roof,
        "mfma": mf,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(synthetic)
    if others:
        out["others"] = others
    print(json.dumps(out))


if __name__ == "__main__":
    main()
