"""HIP-graph capture of the one-call dispatch and of the expert GEMMs: every
replay, with eager work and synchronisations in between and every output
clobbered before it, reproduces the eager result bit for bit."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from tests.gpu_util import DEV, to_dev, to_np
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


def _replay_matches(step, outputs, clobber, reps=4):
    step()
    _sync()
    eager = [to_np(t).copy() for t in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(reps):
        clobber()
        _sync()
        g.replay()
        _sync()
        for i, t in enumerate(outputs):
            assert np.array_equal(to_np(t), eager[i]), (rep, i)


@pytest.mark.parametrize("name,sort", [("decode", 0), ("decode", 1), ("segment", 0), ("segment", 1),
                                       ("prefill", 1), ("mixtral", 1)])
def test_route_dispatch_replays(name, sort):
    """decode unsorted is the identity layout (routing and row copy in one
    launch); the other cases take the counting-sort maps (256-pair chunks
    at the segment-major and Mixtral-like sizes, 512-pair chunks at
    prefill)."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    logits, x = to_dev(inp["logits"]), to_dev(inp["x"])
    xs = None if inp["x_scales"] is None else to_dev(inp["x_scales"])
    n, k, e, g = cfg.n_tokens, cfg.top_k, cfg.n_experts, cfg.n_segments
    ws = torch.empty(moe.moe_route_dispatch_workspace_bytes(n, e, k, g), dtype=torch.uint8, device=DEV)
    idx, w, res = moe.moe_route_dispatch(logits, x, k, g, cfg.renormalize, sort, cfg.sort_cutoff,
                                         x_scales=xs, workspace=ws)
    out = torch.empty((n, cfg.hidden), dtype=torch.bfloat16, device=DEV)

    def step():
        moe.moe_route_dispatch(logits, x, k, g, cfg.renormalize, sort, cfg.sort_cutoff, x_scales=xs,
                               topk_idx=idx, topk_w=w, workspace=ws, out=res)
        if xs is None:
            moe.moe_combine(res.rows, res.dst_pos, w, out=out)

    outputs = [idx, w, res.rows, res.dst_pos, res.src_pair, res.expert_offsets, res.segment_offsets]
    if xs is not None:
        outputs.append(res.row_scales)
    else:
        outputs.append(out)

    def clobber():
        for t in outputs:
            t.zero_()

    _replay_matches(step, outputs, clobber)


def test_grouped_swiglu_replays():
    rng = np.random.default_rng(3)
    e, d, f = 4, 256, 384
    offs = np.array([0, 70, 70, 300, 333], np.int32)
    bits = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(DEV)
    rows = bits(rng.standard_normal((333, d)))
    wg, wu = bits(rng.standard_normal((e, f, d)) * 0.05), bits(rng.standard_normal((e, f, d)) * 0.05)
    wd = bits(rng.standard_normal((e, d, f)) * 0.05)
    offs_d = to_dev(offs)
    y = torch.empty_like(rows)
    ws = torch.empty(moe.moe_grouped_swiglu_workspace_bytes(333, e, d, f), dtype=torch.uint8, device=DEV)
    _replay_matches(lambda: moe.moe_grouped_swiglu(rows, offs_d, wg, wu, wd, y=y, workspace=ws), [y],
                    lambda: y.zero_())


def test_grouped_gemm_fp8_replays():
    rng = np.random.default_rng(4)
    e, k, n = 4, 512, 256
    offs = to_dev(np.array([0, 50, 120, 121, 250], np.int32))
    codes = rng.integers(0, 256, (250, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    wq = rng.integers(0, 256, (e, n, k), dtype=np.uint8)
    wq[(wq & 0x7F) == 0x7F] = 0x30
    rows, w = to_dev(codes), to_dev(wq)
    sx = to_dev(rng.uniform(0.01, 1, (250, k // 128)).astype(np.float32))
    sw = to_dev(rng.uniform(0.01, 1, (e, n // 128, k // 128)).astype(np.float32))
    y = torch.empty((250, n), dtype=torch.bfloat16, device=DEV)
    _replay_matches(lambda: moe.moe_grouped_gemm_fp8(rows, sx, offs, w, sw, y=y), [y], lambda: y.zero_())


def _gather_case(seed=5, e=6, d=256, f=256, r=90):
    rng = np.random.default_rng(seed)
    bits = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(DEV)
    experts = rng.integers(0, e, r).astype(np.int32)
    experts[:20] = 2                                     # one expert with two passes
    rows = bits(rng.standard_normal((r, d)))
    w = (bits(rng.standard_normal((e, f, d)) * 0.05), bits(rng.standard_normal((e, f, d)) * 0.05),
         bits(rng.standard_normal((e, d, f)) * 0.05))
    ws = torch.empty(moe.moe_gather_swiglu_workspace_bytes(r, e, d, f), dtype=torch.uint8, device=DEV)
    return rng, to_dev(experts), rows, w, ws


def test_gather_swiglu_replays():
    """The id grouping, the pass list and both products are recomputed on every
    replay (the workspace is clobbered too)."""
    _, experts, rows, w, ws = _gather_case()
    y = torch.empty_like(rows)
    _replay_matches(lambda: moe.moe_gather_swiglu(rows, experts, *w, y=y, workspace=ws), [y],
                    lambda: (y.zero_(), ws.zero_()))


def test_gather_swiglu_combine_replays():
    """The fused combine adds into out with fp32 atomics in no fixed order, so
    replays are compared with the eager call to fp32 rounding, not bit for bit."""
    rng, experts, rows, w, ws = _gather_case(seed=6, r=96)
    k = 4
    tw = to_dev(rng.uniform(0.1, 1.0, (96 // k, k)).astype(np.float32))
    pairs = to_dev(rng.permutation(96).astype(np.int32))
    out = torch.empty((96 // k, rows.shape[1]), dtype=torch.float32, device=DEV)

    def step():
        out.zero_()
        moe.moe_gather_swiglu_combine(rows, experts, tw, *w, row_pair=pairs, out=out, workspace=ws)

    step()
    _sync()
    eager = to_np(out).astype(np.float64)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(7.0)
        ws.zero_()
        _sync()
        g.replay()
        _sync()
        got = to_np(out).astype(np.float64)
        # terms are O(0.1); a different order of the k fp32 additions moves a sum
        # by a few fp32 ulps of them, a missing term by O(0.1)
        assert np.all(np.abs(got - eager) <= 1e-6 * (np.abs(eager) + 1.0)), rep
