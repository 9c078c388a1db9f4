"""Benchmark of the MoE route -> dispatch -> combine path on one MI355X.

One step = one pass of the hot path over one batch: softmax top-k routing,
dispatch (counts, offsets, stable positions) and the row copy into the
expert-major buffer, identity experts (y = rows), weighted combine back to
token order.  Inputs are resident in HBM before the timed region starts.

Workload (default): prefill, N=4096 tokens, D=7168 bf16, E=256 experts, top-8,
Zipf(1.1) expert popularity, sorted dispatch.  The decode shape (N=128,
unsorted dispatch) is timed in the same run and reported as µs/layer beside
it.

Timing: the K timed steps are captured as one HIP graph of K consecutive
layers (the launch sequence a serving loop replays for a whole forward pass)
and replayed once, bracketed by synchronizations on the wall clock; K replays
of a one-step graph give the figure with a graph launch per layer; K eager
steps with HIP events recorded on the launch stream give the per-stage times
and the dominant kernel's duration.

Output: one JSON line with the whole-path GB/s of algorithmic bytes, a
roofline object for the dominant kernel and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill.json")
KERNEL_SOURCES = {              # kernel -> sources whose hash must match the counters' run
    "scatter": ["combine_moe_route_topk_amd/csrc/dispatch.hip",
                "combine_moe_route_topk_amd/csrc/device_common.hpp"],
    "combine": ["combine_moe_route_topk_amd/csrc/combine.hip",
                "combine_moe_route_topk_amd/csrc/device_common.hpp"],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "decode", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-all", action="store_true", help="skip the five-workload table")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--calib-copy", action="store_true",
                    help="run only a plain device copy of known size (PMC counter calibration)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="run only torch's bf16 linear (hipBLASLt) on the Mixtral-like layer's "
                         "dense and per-expert products, for comparison with the grouped SwiGLU")
    ap.add_argument("--crossover", action="store_true",
                    help="run only the sorted/unsorted crossover table of the decode layer "
                         "with SwiGLU experts over a range of token counts")
    return ap.parse_args()


# ------------------------------------------------------------------ bytes per step

def algorithmic_bytes(n, d, e, k, g, elem):
    nk = n * k
    route = n * e * 4 + 2 * nk * 4
    maps = nk * 4 + 3 * nk * 4 + (e + (e + 1) + (g + 1)) * 4
    scatter = n * d * elem + nk * d * elem + nk * 4
    combine = nk * d * elem + 2 * nk * 4 + n * d * elem
    return dict(route=route, maps=maps, scatter=scatter, combine=combine,
                total=route + maps + scatter + combine)


def source_sha(rels):
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ GPU side

class Path:
    """Preallocated buffers and the calls of one step.

    split=False: moe_route_dispatch with the payload | moe_combine (the step
                 every bench leg times);
    split=True:  moe_route_dispatch (maps only) | moe_scatter_rows | moe_combine,
                 which puts the row copy in a launch of its own between events."""

    def __init__(self, cfg, torch, moe, split=True):
        from workloads import make_inputs
        self.torch, self.moe, self.cfg, self.split = torch, moe, cfg, split
        dev = torch.device("cuda:0")
        inp = make_inputs(cfg)
        self.inputs = inp
        n, d, e, k, g = cfg.n_tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.n_segments
        self.logits = torch.from_numpy(inp["logits"]).to(dev)
        if cfg.dtype == "bf16":
            self.x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        elif cfg.dtype == "f32":
            self.x = torch.from_numpy(inp["x"]).to(dev)
        else:
            raise ValueError("bench workloads carry bf16 or fp32 payloads")
        self.out = torch.empty((n, d), dtype=self.x.dtype, device=dev)
        self.ws = torch.empty(moe.moe_route_dispatch_workspace_bytes(n, e, k, g), dtype=torch.uint8,
                              device=dev)
        self.sort = cfg.sort if cfg.sort in (-1, 0, 1) else 1
        self.idx, self.w, self.res = moe.moe_route_dispatch(
            self.logits, None if split else self.x, k, g, cfg.renormalize, self.sort,
            cfg.sort_cutoff, workspace=self.ws)
        self.rows = torch.empty((n * k, d), dtype=self.x.dtype, device=dev) if split else self.res.rows
        self.stream = torch.cuda.current_stream()

    def step(self, ev=None):
        moe, c = self.moe, self.cfg
        if ev: ev[0].record(self.stream)
        moe.moe_route_dispatch(self.logits, None if self.split else self.x, c.top_k, c.n_segments,
                               c.renormalize, self.sort, c.sort_cutoff, topk_idx=self.idx,
                               topk_w=self.w, workspace=self.ws, out=self.res)
        if ev: ev[1].record(self.stream)
        if self.split:
            moe.moe_scatter_rows(self.x, self.res.dst_pos, c.top_k, rows=self.rows)
        if ev: ev[2].record(self.stream)
        moe.moe_combine(self.rows, self.res.dst_pos, self.w, out=self.out)
        if ev: ev[3].record(self.stream)


def time_path(path, steps, warmup):
    torch = path.torch
    for _ in range(warmup):
        path.step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        path.step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)] for i in range(steps)])
    return wall / steps * 1e3, stage.mean(axis=0) * 1e3, np.median(stage, axis=0) * 1e3


def capture(torch, step, n):
    """n consecutive calls of step() captured in one HIP graph (torch.cuda.CUDAGraph)."""
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            step()
    return g


def graph_times(torch, step, steps, warmup, replays=11):
    """Per-step wall time of the step in HIP graphs, in ms.

    Timed steps: K consecutive steps captured as one graph, the way a serving
    loop captures a whole forward pass of K layers, replayed `replays` times,
    each replay between two synchronizations on the wall clock.  Untimed
    before it: W replays of a one-step graph, then one replay of the K-step
    graph (its one-time upload to the device).  The one-step graph is also
    timed over K replays: that figure includes the launch of a graph per step.
    Returns ({p10, p50, p90} of the K-step graph's per-step time over the
    replays, one-step graph)."""
    g1 = capture(torch, step, 1)
    for _ in range(warmup):
        g1.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g1.replay()
    torch.cuda.synchronize()
    one = (time.perf_counter() - t0) / steps * 1e3
    gk = capture(torch, step, steps)
    gk.replay()
    torch.cuda.synchronize()
    per_step = []
    for _ in range(replays):
        t0 = time.perf_counter()
        gk.replay()
        torch.cuda.synchronize()
        per_step.append((time.perf_counter() - t0) / steps * 1e3)
    del gk, g1
    return pct(per_step), one


def pct(values):
    """{p10, p50, p90} of a list of timings."""
    v = np.asarray(values, dtype=np.float64)
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
            "p90": float(np.percentile(v, 90)), "n": int(v.size)}


def cold_times(torch, step, reps=21, flush_bytes=1 << 30):
    """Per-step time with cold caches, in ms: before every timed step, untimed,
    an elementwise pass reads and writes a 1 GiB buffer (4x the 256 MB
    last-level cache), so the step's inputs come from HBM.  Each step is a
    one-step graph replay timed with HIP events on the launch stream (the
    flush is queued ahead of them, so no launch gap is timed)."""
    flush = torch.zeros(flush_bytes // 4, dtype=torch.float32, device="cuda:0")
    g1 = capture(torch, step, 1)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        flush.add_(1.0)
        e0.record(stream)
        g1.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    out = pct([e0.elapsed_time(e1) for e0, e1 in evs])
    del flush, g1
    return out


def check_outputs(path):
    """Spot-check the timed buffers against the oracle (a few tokens)."""
    from oracle import codecs
    from oracle.combine import combine_f64
    from oracle.route import route_topk
    torch, c = path.torch, path.cfg
    torch.cuda.synchronize()
    oi, _ = route_topk(path.inputs["logits"], c.top_k, c.renormalize)
    if not np.array_equal(path.idx.cpu().numpy(), oi):
        raise RuntimeError("routing indices of the timed run differ from the oracle")
    toks = np.linspace(0, c.n_tokens - 1, 8).astype(int)
    dst = path.res.dst_pos.cpu().numpy()
    w = path.w.cpu().numpy()
    xf = codecs.bf16_bits_to_f32(path.inputs["x"]) if c.dtype == "bf16" else path.inputs["x"]
    rows_f = np.zeros((c.n_tokens * c.top_k, c.hidden), np.float32)
    for t in toks:
        for j in range(c.top_k):
            rows_f[dst[t * c.top_k + j]] = xf[t]
    exact = combine_f64(rows_f, dst, w, c.top_k, tokens=toks)
    got = path.out[torch.from_numpy(toks).to(path.out.device)].float().cpu().numpy()
    if not np.all(np.abs(got - exact) <= 2.0 ** -7 * np.abs(exact) + 1e-30):
        raise RuntimeError("combine output of the timed run differs from the oracle")


def expert_load(res):
    """Realised rows per expert of a dispatch: the histogram's extremes."""
    c = res.expert_counts.cpu().numpy()
    return {"max": int(c.max()), "min": int(c.min()), "mean": round(float(c.mean()), 2),
            "empty_experts": int((c == 0).sum()), "top4": sorted(c.tolist())[-4:][::-1]}


def dc_bytes(cfg):
    """Algorithmic bytes of route + dispatch + combine for any workload (fp8
    payloads move one byte per element plus their fp32 block scales; the
    combine reads bf16 expert outputs)."""
    n, d, e, k, g = cfg.n_tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.n_segments
    nk = n * k
    b = algorithmic_bytes(n, d, e, k, g, cfg.elem_bytes)
    if cfg.dtype == "f8":
        sc = d // 128 * 4
        b["scatter"] += (n + nk) * sc
        b["combine"] = nk * d * 2 + 2 * nk * 4 + n * d * 2
        b["total"] = b["route"] + b["maps"] + b["scatter"] + b["combine"]
    return b


def time_all_configs(torch, moe, steps, warmup):
    """route -> dispatch (maps and rows) -> combine for each of the five
    workloads, timed as in graph_times (K consecutive steps in one graph; the
    one-step graph's figure beside it).  Expert outputs are an
    input of the combine: identity experts read the dispatched rows; the fp8
    workload's identity expert (dequantisation to bf16) runs once before the
    timing.  The segment-major workload alternates the sort flag per call, so
    its step is two calls (unsorted, then sorted) and the figure is per call."""
    from workloads import CONFIGS, make_inputs
    dev = torch.device("cuda:0")
    out = {}
    for name, cfg in CONFIGS.items():
        inp = make_inputs(cfg)
        logits = torch.from_numpy(inp["logits"]).to(dev)
        if cfg.dtype == "bf16":
            x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
        elif cfg.dtype == "f32":
            x = torch.from_numpy(inp["x"]).to(dev)
        else:
            x = torch.from_numpy(inp["x"]).to(dev)
        xs = torch.from_numpy(inp["x_scales"]).to(dev) if inp["x_scales"] is not None else None
        n, k, e, g = cfg.n_tokens, cfg.top_k, cfg.n_experts, cfg.n_segments
        sorts = [0, 1] if cfg.sort == "alternate" else [cfg.sort]
        ws = torch.empty(moe.moe_route_dispatch_workspace_bytes(n, e, k, g), dtype=torch.uint8, device=dev)
        idx, w, res = moe.moe_route_dispatch(logits, x, k, g, cfg.renormalize, sorts[0], cfg.sort_cutoff,
                                             x_scales=xs, workspace=ws)
        y = moe.moe_dequant_rows(res.rows, res.row_scales) if cfg.dtype == "f8" else res.rows
        o = torch.empty((n, cfg.hidden), dtype=y.dtype, device=dev)

        def step():
            for srt in sorts:
                moe.moe_route_dispatch(logits, x, k, g, cfg.renormalize, srt, cfg.sort_cutoff,
                                       x_scales=xs, topk_idx=idx, topk_w=w, workspace=ws, out=res)
                moe.moe_combine(y, res.dst_pos, w, out=o)

        reps = max(steps, 50)
        ms_k, ms_1 = graph_times(torch, step, reps, warmup)
        us = ms_k["p50"] * 1e3 / len(sorts)
        us1 = ms_1 * 1e3 / len(sorts)
        b = dc_bytes(cfg)["total"]
        out[name] = {"us_per_layer": round(us, 2),
                     "us_per_layer_p10_p90": [round(ms_k["p10"] * 1e3 / len(sorts), 2),
                                              round(ms_k["p90"] * 1e3 / len(sorts), 2)],
                     "us_per_layer_graph1": round(us1, 2),
                     "GB_per_s": round(b / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "bytes": b, "mode": "alternating unsorted/sorted" if len(sorts) > 1 else
                     ("sorted" if res.sorted else "unsorted")}
        del x, xs, y, o, res, ws, logits
    return out


def time_swiglu(torch, moe, steps=10, warmup=2, cpu=False):
    """The Mixtral-like layer's grouped SwiGLU (N=8192, k=2 -> 16384 rows,
    D=4096, F=14336, E=8) reading the sorted dispatch in place."""
    from workloads import CONFIGS, make_inputs, make_swiglu_weights_device
    cfg = CONFIGS["mixtral"]
    inp = make_inputs(cfg)
    dev = torch.device("cuda:0")
    w = make_swiglu_weights_device(cfg)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    idx, tw = moe.moe_route_topk(logits, cfg.top_k)
    res = moe.moe_dispatch(x, idx, cfg.n_experts, 1, sort=-1, sort_cutoff=cfg.sort_cutoff)
    rows = res.rows.shape[0]
    ws = torch.empty(moe.moe_grouped_swiglu_workspace_bytes(rows, cfg.n_experts, cfg.hidden, cfg.ffn),
                     dtype=torch.uint8, device=dev)
    y = torch.empty_like(res.rows)
    call = lambda: moe.moe_grouped_swiglu(res.rows, res.expert_offsets, w["w_gate"], w["w_up"],
                                          w["w_down"], y=y, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = 2.0 * rows * cfg.hidden * cfg.ffn * 3
    tflops = flop / (ms * 1e-3) / 1e12
    out = {"workload": f"mixtral: {cfg.note}", "rows": rows, "ms": round(ms, 3),
           "tflops": round(tflops, 1), "peak_tflops": 2500.0, "frac": round(tflops / 2500.0, 4),
           "flop": flop, "dtype": "bf16 in, fp32 accumulate"}
    if cpu:
        out["cpu_oracle"] = cpu_oracle_swiglu(torch, res, w)
    return out


def time_fp8_gemm(torch, moe, steps=10, warmup=2, cpu=False):
    """The segment-major workload's fp8 expert projection (N_out = 4096, K =
    7168, 256 experts): the sorted fp8 dispatch's rows and 1x128 scales read in
    place by the block-scaled grouped GEMM.  Weight streaming dominates."""
    from workloads import CONFIGS, FP8_GEMM_N, make_fp8_expert_weights_device, make_inputs
    cfg = CONFIGS["segment"]
    inp = make_inputs(cfg)
    dev = torch.device("cuda:0")
    x = torch.from_numpy(inp["x"]).to(dev)
    xs = torch.from_numpy(inp["x_scales"]).to(dev)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    _, _, res = moe.moe_route_dispatch(logits, x, cfg.top_k, cfg.n_segments, cfg.renormalize, 1,
                                       cfg.sort_cutoff, x_scales=xs)
    wt = make_fp8_expert_weights_device(cfg)
    rows = res.rows.shape[0]
    n, k, e = FP8_GEMM_N, cfg.hidden, cfg.n_experts
    y = torch.empty((rows, n), dtype=torch.bfloat16, device=dev)
    call = lambda: moe.moe_grouped_gemm_fp8(res.rows, res.row_scales, res.expert_offsets, wt["w"],
                                            wt["w_scales"], y=y)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    counts = res.expert_counts.cpu().numpy()
    active = int((counts > 0).sum())
    wbytes = active * (n * k + (n // 128) * (k // 128) * 4)
    b = wbytes + rows * (k + (k // 128) * 4) + rows * n * 2 + (e + 1) * 4
    gbs = b / (ms * 1e-3) / 1e9
    flop = 2.0 * rows * n * k
    out = {"workload": f"segment: {cfg.note}; fp8 projection N={n} read in place", "rows": rows,
           "active_experts": active, "ms": round(ms, 3), "bytes": b, "weight_bytes": wbytes,
           "GB_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "tflops": round(flop / (ms * 1e-3) / 1e12, 1), "flop": flop,
           "bound": "hbm (weights)", "dtype": "fp8 e4m3fn in, fp32 accumulate, bf16 out"}
    if cpu:
        out["cpu_oracle"] = cpu_oracle_fp8_gemm(torch, res, wt)
    del wt, y, res, x, xs
    torch.cuda.empty_cache()
    return out


def time_gather_swiglu(torch, moe, steps=10, warmup=2, cpu=False):
    """Decode with real experts (N=128, D=7168, E=256, top-8, F=2048): the
    unsorted identity-layout rows read where the dispatch left them by the
    per-row-expert SwiGLU.  Every active expert's three [F, D] matrices are
    streamed once, which dominates the bytes.  Timed alone and as the whole
    layer (route + unsorted dispatch + expert FFN + combine)."""
    from workloads import DECODE_FFN, make_inputs, make_swiglu_weights_device
    cfg = DECODE_FFN
    inp = make_inputs(cfg)
    dev = torch.device("cuda:0")
    w = make_swiglu_weights_device(cfg)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    idx, tw, res = moe.moe_route_dispatch(logits, x, cfg.top_k, cfg.n_segments, cfg.renormalize,
                                          cfg.sort, cfg.sort_cutoff)
    rows = res.rows.shape[0]
    e, d, f = cfg.n_experts, cfg.hidden, cfg.ffn
    ws = torch.empty(moe.moe_gather_swiglu_workspace_bytes(rows, e, d, f), dtype=torch.uint8,
                     device=dev)
    y = torch.empty_like(res.rows)
    ffn = lambda: moe.moe_gather_swiglu(res.rows, res.row_expert, w["w_gate"], w["w_up"],
                                        w["w_down"], y=y, workspace=ws)
    rd_ws = torch.empty(moe.moe_route_dispatch_workspace_bytes(cfg.n_tokens, e, cfg.top_k, 1),
                        dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)

    def layer():
        moe.moe_route_dispatch(logits, x, cfg.top_k, cfg.n_segments, cfg.renormalize, cfg.sort,
                               cfg.sort_cutoff, topk_idx=idx, topk_w=tw, workspace=rd_ws, out=res)
        ffn()
        moe.moe_combine(y, res.dst_pos, tw, out=out)

    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    out32 = torch.empty((cfg.n_tokens, d), dtype=torch.float32, device=dev)

    def layer_fused():
        moe.moe_route_dispatch(logits, x, cfg.top_k, cfg.n_segments, cfg.renormalize, cfg.sort,
                               cfg.sort_cutoff, topk_idx=idx, topk_w=tw, workspace=rd_ws, out=res)
        out32.zero_()
        moe.moe_gather_swiglu_combine(res.rows, res.row_expert, tw, w["w_gate"], w["w_up"],
                                      w["w_down"], row_pair=res.src_pair, out=out32, workspace=ws)

    ms = timed(ffn)
    ms_layer = timed(layer)
    ms_fused = timed(layer_fused)
    counts = res.expert_counts.cpu().numpy()
    active = int((counts > 0).sum())
    wbytes = active * 3 * f * d * 2
    b = wbytes + rows * d * 2 + rows * 4 + 2 * rows * f * 2 + rows * d * 2
    gbs = b / (ms * 1e-3) / 1e9
    rec = {"workload": f"decode_ffn: {cfg.note}", "rows": rows, "active_experts": active,
           "max_rows_per_expert": int(counts.max()), "ms": round(ms, 3), "bytes": b,
           "weight_bytes": wbytes, "GB_per_s": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "layer_ms": round(ms_layer, 3),
           "layer_calls": "moe_route_dispatch (unsorted, with rows) + moe_gather_swiglu + moe_combine",
           "layer_fused_ms": round(ms_fused, 3),
           "layer_fused_calls": "moe_route_dispatch + zero fill of the fp32 out + "
                                "moe_gather_swiglu_combine (combine fused into the down product)",
           "bound": "hbm (weights)", "dtype": "bf16 in, fp32 accumulate, bf16 out"}
    if cpu:
        rec["cpu_oracle"] = cpu_oracle_gather_swiglu(torch, res, w)
    del w, y, ws, res, x, logits, out32
    torch.cuda.empty_cache()
    return rec


# ------------------------------------------------------------------ CPU baseline

def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def _time_oracle(fn, min_seconds=10.0, max_repeats=200):
    times = []
    while len(times) < max_repeats and (len(times) < 1 or sum(times) < min_seconds):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times), sum(times)


def cpu_oracle_swiglu(torch, res, w, n_sample=128):
    """The oracle's SwiGLU on the first rows of expert 0 (its weights copied
    back from the device), timed on the host."""
    from oracle.swiglu import swiglu_rows
    offs = res.expert_offsets.cpu().numpy()
    m = int(min(n_sample, offs[1] - offs[0]))
    rows = res.rows[int(offs[0]):int(offs[0]) + m].view(torch.int16).cpu().numpy().view(np.uint16)
    host = {k: v[0:1].view(torch.int16).cpu().numpy().view(np.uint16) for k, v in w.items()}
    experts = np.zeros(m, np.int64)
    dt, n, tot = _time_oracle(lambda: swiglu_rows(rows, experts, host["w_gate"], host["w_up"], host["w_down"]))
    f, d = host["w_gate"].shape[1], host["w_gate"].shape[2]
    return dict(value=round(2.0 * m * d * 3 * f / dt / 1e12, 5), unit="TFLOP/s", cores=_blas_threads(),
                kind="oracle", sample=f"{m} rows of expert 0, float64 numpy (BLAS matmul); median of {n} "
                                      f"passes ({tot:.1f} s)", seconds_per_pass=round(dt, 3))


def cpu_oracle_fp8_gemm(torch, res, wt, n_experts_sample=2):
    """The oracle's fp8 block-scaled GEMM on every row of the first experts
    that own rows (their weights copied back), timed on the host; GB/s of the
    sample's algorithmic bytes."""
    from oracle.gemm_fp8 import gemm_fp8_rows
    offs = res.expert_offsets.cpu().numpy()
    busy = [e for e in range(offs.size - 1) if offs[e + 1] > offs[e]][:n_experts_sample]
    sel = np.concatenate([np.arange(offs[e], offs[e + 1]) for e in busy])
    experts = np.concatenate([np.full(offs[e + 1] - offs[e], j) for j, e in enumerate(busy)])
    rows = res.rows.cpu().numpy()[sel]
    sx = res.row_scales.cpu().numpy()[sel]
    idx = torch.tensor(busy, device=wt["w"].device)
    w = wt["w"].index_select(0, idx).cpu().numpy()
    sw = wt["w_scales"].index_select(0, idx).cpu().numpy()
    dt, n, tot = _time_oracle(lambda: gemm_fp8_rows(rows, sx, experts, w, sw))
    nn, k = w.shape[1], w.shape[2]
    b = len(busy) * (nn * k + sw[0].size * 4) + sel.size * (k + sx.shape[1] * 4) + sel.size * nn * 2
    return dict(value=round(b / dt / 1e9, 4), unit="GB/s", cores=_blas_threads(), kind="oracle",
                sample=f"all {sel.size} rows of experts {busy}, float64 numpy; median of {n} passes "
                       f"({tot:.1f} s)", seconds_per_pass=round(dt, 3))


def cpu_oracle_gather_swiglu(torch, res, w, n_experts_sample=2):
    """The oracle's row-by-row SwiGLU on every row of the first experts that
    own rows (their weights copied back), timed on the host; GB/s of the
    sample's algorithmic bytes."""
    from oracle.swiglu import swiglu_rows
    rexp = res.row_expert.cpu().numpy()
    busy = np.unique(rexp)[:n_experts_sample]
    sel = np.nonzero(np.isin(rexp, busy))[0]
    rows = res.rows.view(torch.int16).cpu().numpy().view(np.uint16)[sel]
    local = np.searchsorted(busy, rexp[sel])
    idx = torch.tensor(busy, device=w["w_gate"].device)
    host = {k: v.index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
            for k, v in w.items()}
    dt, n, tot = _time_oracle(lambda: swiglu_rows(rows, local, host["w_gate"], host["w_up"],
                                                  host["w_down"]))
    f, d = host["w_gate"].shape[1], host["w_gate"].shape[2]
    b = len(busy) * 3 * f * d * 2 + sel.size * (d * 2 + 4 + 2 * f * 2 + d * 2)
    return dict(value=round(b / dt / 1e9, 4), unit="GB/s", cores=_blas_threads(), kind="oracle",
                sample=f"all {sel.size} rows of experts {busy.tolist()}, float64 numpy; median "
                       f"of {n} passes ({tot:.1f} s)", seconds_per_pass=round(dt, 3))


def cpu_baseline(cfg, n_sample, min_seconds=10.0, max_repeats=20):
    """The oracle as it stands, on the first ``n_sample`` tokens of the same
    workload, repeated until ~min_seconds of CPU work; median pass time."""
    from oracle import codecs, dispatch as od
    from oracle.combine import combine_f64
    from oracle.route import route_topk
    from workloads import make_inputs
    sub = cfg.with_tokens(min(n_sample, cfg.n_tokens))
    inp = make_inputs(sub)
    times = []
    while len(times) < max_repeats and (len(times) < 1 or sum(times) < min_seconds):
        t0 = time.perf_counter()
        idx, w = route_topk(inp["logits"], sub.top_k, sub.renormalize)
        sorted_ = od.resolve_sorted(cfg.sort if cfg.sort in (-1, 0, 1) else 1, sub.n_tokens,
                                    sub.sort_cutoff)
        res = od.dispatch(idx, sub.n_experts, sub.n_segments, sorted_, x=inp["x"])
        y = codecs.bf16_bits_to_f32(res["rows"]) if sub.dtype == "bf16" else res["rows"]
        out = combine_f64(y, res["dst_pos"], w, sub.top_k)
        if sub.dtype == "bf16":
            codecs.f64_to_bf16_bits(out)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    b = algorithmic_bytes(sub.n_tokens, sub.hidden, sub.n_experts, sub.top_k, sub.n_segments,
                          sub.elem_bytes)["total"]
    return dict(value=round(b / dt / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"{sub.n_tokens} of {cfg.n_tokens} tokens of the same workload; median of "
                       f"{len(times)} passes of route+dispatch+combine ({sum(times):.1f} s total, "
                       "numpy, single-threaded)",
                seconds_per_pass=round(dt, 3))


# ------------------------------------------------------------------ main

def calib_copy(torch):
    """A plain device copy of 1 GiB, for scaling FETCH_SIZE / WRITE_SIZE."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": n, "launches": 5}))


def library_gemm(torch, reps=10):
    """torch's bf16 linear (hipBLASLt on ROCm) on the products of the
    Mixtral-like layer (16384 rows, D=4096, F=14336, 8 experts of ~2048 rows):
    the gate and up projections as one dense [16384, 4096] x [4096, 28672]
    product and the down projection as [16384, 14336] x [14336, 4096], and the
    same per expert (2048 rows).  Activations N(0, 1), weights N(0, 0.02), as
    in the workload (the matrix cores' power depends on the data)."""
    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    stream = torch.cuda.current_stream()
    rec = {}
    for name, m, n, k in (("dense_gate_up", 16384, 28672, 4096), ("dense_down", 16384, 4096, 14336),
                          ("expert_gate_up", 2048, 28672, 4096), ("expert_down", 2048, 4096, 14336)):
        a = torch.randn((m, k), device=dev, generator=gen).to(torch.bfloat16)
        w = (torch.randn((n, k), device=dev, generator=gen) * 0.02).to(torch.bfloat16)
        for _ in range(3):
            out = torch.nn.functional.linear(a, w)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            out = torch.nn.functional.linear(a, w)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rec[name] = {"m": m, "n": n, "k": k, "ms": round(ms, 4),
                     "tflops": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1)}
        del a, w, out
    layer = rec["dense_gate_up"]["ms"] + rec["dense_down"]["ms"]
    per_expert = 8 * (rec["expert_gate_up"]["ms"] + rec["expert_down"]["ms"])
    flop = 2.0 * 16384 * 4096 * 14336 * 3
    rec["layer_dense_ms"] = round(layer, 3)
    rec["layer_dense_tflops"] = round(flop / (layer * 1e-3) / 1e12, 1)
    rec["layer_8_expert_calls_ms"] = round(per_expert, 3)
    rec["layer_8_expert_calls_tflops"] = round(flop / (per_expert * 1e-3) / 1e12, 1)
    print(json.dumps({"library_gemm": rec, "what": "torch.nn.functional.linear bf16 (hipBLASLt), "
                      "HIP events over 10 calls after 3 warm-up calls"}), flush=True)


def crossover(torch, moe, steps=5, warmup=2):
    """The sorted/unsorted switch measured on MoE layers with SwiGLU experts
    over a range of token counts: each layer is route + dispatch + expert FFN
    + combine, K steps in one graph.
      unsorted+gather: identity layout, per-row-expert FFN (moe_gather_swiglu)
      sorted+grouped:  expert-major layout, grouped FFN (moe_grouped_swiglu)
      sorted+gather:   expert-major layout, per-row-expert FFN
    and with identity experts (route + dispatch + combine) in both modes.
    Two expert shapes: the decode workload's (D=7168, E=256, top-8, F=2048)
    and the Mixtral-like one (D=4096, E=8, top-2, F=14336)."""
    from workloads import CONFIGS, DECODE_FFN, make_inputs, make_swiglu_weights_device
    dev = torch.device("cuda:0")
    result = {}
    for base, ns in ((DECODE_FFN, (16, 32, 64, 128, 256, 512, 640, 768, 896, 1024, 2048)),
                     (CONFIGS["mixtral"], (8, 16, 32, 64, 128, 256, 512))):
        w = make_swiglu_weights_device(base)
        e, d, f, k = base.n_experts, base.hidden, base.ffn, base.top_k
        table = []
        for n in ns:
            cfg = base.with_tokens(n)
            inp = make_inputs(cfg)
            logits = torch.from_numpy(inp["logits"]).to(dev)
            x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
            rd_ws = torch.empty(moe.moe_route_dispatch_workspace_bytes(n, e, k, 1),
                                dtype=torch.uint8, device=dev)
            gws = torch.empty(moe.moe_gather_swiglu_workspace_bytes(n * k, e, d, f),
                              dtype=torch.uint8, device=dev)
            sws = torch.empty(moe.moe_grouped_swiglu_workspace_bytes(n * k, e, d, f),
                              dtype=torch.uint8, device=dev)
            y = torch.empty((n * k, d), dtype=torch.bfloat16, device=dev)
            out = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
            row = {"n_tokens": n, "rows_per_expert": round(n * k / e, 2)}
            for mode in ("unsorted+gather", "sorted+grouped", "sorted+gather",
                         "identity unsorted", "identity sorted"):
                sort = 0 if mode in ("unsorted+gather", "identity unsorted") else 1
                idx, tw, res = moe.moe_route_dispatch(logits, x, k, 1, True, sort, 256,
                                                      workspace=rd_ws)

                def step(sort=sort, mode=mode, idx=idx, tw=tw, res=res):
                    moe.moe_route_dispatch(logits, x, k, 1, True, sort, 256, topk_idx=idx,
                                           topk_w=tw, workspace=rd_ws, out=res)
                    if mode.endswith("gather"):
                        moe.moe_gather_swiglu(res.rows, res.row_expert, w["w_gate"], w["w_up"],
                                              w["w_down"], y=y, workspace=gws)
                        moe.moe_combine(y, res.dst_pos, tw, out=out)
                    elif mode.endswith("grouped"):
                        moe.moe_grouped_swiglu(res.rows, res.expert_offsets, w["w_gate"],
                                               w["w_up"], w["w_down"], y=y, workspace=sws)
                        moe.moe_combine(y, res.dst_pos, tw, out=out)
                    else:
                        moe.moe_combine(res.rows, res.dst_pos, tw, out=out)

                gk, _ = graph_times(torch, step, steps if "identity" not in mode else 50, warmup,
                                    replays=5)
                row[mode] = round(gk["p50"] * 1e3, 2)
                del res, idx, tw
            table.append(row)
            print(json.dumps({base.name: row}), flush=True)
            del logits, x, rd_ws, gws, sws, y, out
        del w
        torch.cuda.empty_cache()
        cross = [r["n_tokens"] for r in table if r["sorted+grouped"] < r["unsorted+gather"]]
        result[base.name] = {"table": table,
                             "first_n_where_sorted_grouped_wins": cross[0] if cross else None,
                             "shape": f"D={base.hidden}, E={base.n_experts}, top-{base.top_k}, "
                                      f"F={base.ffn}"}
    print(json.dumps({"crossover": result, "unit": "us per layer (median of 5 replays of a "
                      "K-step graph)"}), flush=True)


def copy_ceiling(torch, nbytes, reps=10):
    """A plain device copy moving the same bytes as one step (half read, half
    written), timed with HIP events: the copy ceiling the path is compared with."""
    half = nbytes // 2 // 16 * 16
    a = torch.empty(half, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return {"GB_per_s": round(2 * half / (ms * 1e-3) / 1e9, 1), "bytes_moved": 2 * half,
            "what": "torch device-to-device copy of half the step's bytes (read + write)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is timed on a single GPU's share of the work)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    if args.calib_copy:
        calib_copy(torch)
        return
    if args.library_gemm:
        library_gemm(torch)
        return
    import combine_moe_route_topk_amd as moe
    if args.crossover:
        crossover(torch, moe)
        return
    from workloads import CONFIGS

    cfg = CONFIGS[args.workload]
    path = Path(cfg, torch, moe, split=False)
    ms_eager, stage_mean_us, stage_med_us = time_path(path, args.steps, args.warmup)
    check_outputs(path)
    gk, ms_g1 = graph_times(torch, path.step, args.steps, args.warmup)   # the timed steps
    ms = gk["p50"]
    check_outputs(path)
    cold = cold_times(torch, path.step)
    check_outputs(path)
    n, d, e, k, g = cfg.n_tokens, cfg.hidden, cfg.n_experts, cfg.top_k, cfg.n_segments
    b = algorithmic_bytes(n, d, e, k, g, cfg.elem_bytes)
    value = b["total"] / (ms * 1e-3) / 1e9
    ceiling = copy_ceiling(torch, b["total"])

    # one call routes and dispatches (maps and rows); the combine is the other
    stages = {"route+dispatch": float(stage_mean_us[0] + stage_mean_us[1]),
              "combine": float(stage_mean_us[2])}
    dom = "combine"
    achieved = b[dom] / (stages[dom] * 1e-6) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        ent = tr.get(dom)
        if ent and ent.get("source_sha") == source_sha(KERNEL_SOURCES[dom]) and tr.get("workload") == args.workload:
            traffic = ent["hbm_bytes_per_launch"]
    roofline = dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    algorithmic_bytes=b[dom], avg_us=round(stages[dom], 2))

    rec = {
        "metric": "dispatch+combine µs/layer and HBM GB/s (% peak) at 128 and 4096 tokens",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.note}", "n_tokens": n, "hidden": d,
                   "n_experts": e, "top_k": k, "n_segments": g,
                   "sort": "sorted" if path.res.sorted else "unsorted", "experts": "identity",
                   "bytes_per_step": b["total"], "expert_load": expert_load(path.res)},
        "timing": "K consecutive steps captured as one HIP graph (a K-layer forward pass), "
                  "replayed 11 times, wall clock between synchronizations around each replay; "
                  "value and ms_per_step from the median replay; graph1 = K replays of a "
                  "one-step graph; cold = one-step graph after a 1 GiB read+write flush, HIP "
                  "events; stages from HIP events over K eager steps",
        "us_per_layer": round(ms * 1e3, 2),
        "us_per_layer_pct": {q: round(v * 1e3, 2) for q, v in gk.items() if q != "n"},
        "us_per_layer_cold": {q: round(v * 1e3, 2) for q, v in cold.items() if q != "n"},
        "us_per_layer_graph1": round(ms_g1 * 1e3, 2),
        "us_per_layer_eager": round(ms_eager * 1e3, 2),
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "copy_ceiling": ceiling,
        "frac_of_copy_ceiling": round(value / ceiling["GB_per_s"], 4),
        "stages_us": {nm: round(v, 2) for nm, v in stages.items()},
        "calls": "moe_route_dispatch (routing, maps and rows) + moe_combine",
        "roofline": roofline,
    }
    if not args.no_decode and args.workload == "prefill":
        dcfg = CONFIGS["decode"]
        dpath = Path(dcfg, torch, moe, split=False)
        dms, dst_us, _ = time_path(dpath, max(args.steps, 200), args.warmup)
        check_outputs(dpath)
        db = algorithmic_bytes(dcfg.n_tokens, dcfg.hidden, dcfg.n_experts, dcfg.top_k,
                               dcfg.n_segments, dcfg.elem_bytes)
        dk, gms1 = graph_times(torch, dpath.step, max(args.steps, 200), args.warmup)
        gms = dk["p50"]
        check_outputs(dpath)
        dcold = cold_times(torch, dpath.step)
        check_outputs(dpath)
        rec["decode"] = {"workload": f"decode: {dcfg.note}", "us_per_layer": round(gms * 1e3, 2),
                         "us_per_layer_pct": {q: round(v * 1e3, 2) for q, v in dk.items() if q != "n"},
                         "us_per_layer_cold": {q: round(v * 1e3, 2) for q, v in dcold.items() if q != "n"},
                         "us_per_layer_graph1": round(gms1 * 1e3, 2),
                         "us_per_layer_eager": round(dms * 1e3, 2),
                         "calls": "moe_route_dispatch (with rows) + moe_combine",
                         "GB_per_s": round(db["total"] / (gms * 1e-3) / 1e9, 1),
                         "cache": "us_per_layer: hot (the step's 33 MB of buffers can stay in the "
                                  "256 MB last-level cache between steps); us_per_layer_cold: "
                                  "1 GiB flush before every step",
                         "stages_us": {"route+dispatch": round(float(dst_us[0] + dst_us[1]), 2),
                                       "combine": round(float(dst_us[2]), 2)}}
    if not args.no_all and args.workload == "prefill":
        rec["all_configs"] = time_all_configs(torch, moe, args.steps, args.warmup)
    if not args.no_gemm and args.workload == "prefill":
        rec["grouped_swiglu"] = time_swiglu(torch, moe, cpu=not args.no_cpu_baseline)
        torch.cuda.empty_cache()
        rec["grouped_gemm_fp8"] = time_fp8_gemm(torch, moe, cpu=not args.no_cpu_baseline)
        torch.cuda.empty_cache()
        rec["gather_swiglu"] = time_gather_swiglu(torch, moe, cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_tokens)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
