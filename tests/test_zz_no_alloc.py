"""The allocation-free route + dispatch (moe_route_dispatch_noalloc: the
chunk histograms live in the library's static per-GPU scratch array) against
moe_route_dispatch with a caller workspace, through the C ABI.  The two share
their kernels, so every output must be bit-identical.  Each case makes two
calls in a row, the second with a smaller input, so the second call runs on
scratch that still holds the first call's contents."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from tests.gpu_util import DEV, to_dev
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

FIELDS = ("expert_counts", "expert_offsets", "segment_offsets", "src_pair", "dst_pos", "row_expert",
          "rows", "row_scales")


def _bits(t):
    if t is None:
        return None
    t = t.contiguous()
    if t.dtype in (torch.bfloat16, torch.float32):
        t = t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
    return t.cpu().numpy()


def _inputs(name, n_tokens=None):
    cfg = CONFIGS[name] if n_tokens is None else CONFIGS[name].with_tokens(n_tokens)
    inp = make_inputs(cfg)
    xs = None if inp["x_scales"] is None else to_dev(inp["x_scales"])
    return cfg, to_dev(inp["logits"]), to_dev(inp["x"]), xs


def _random_inputs(n, e, d, seed):
    rng = np.random.default_rng(seed)
    logits = torch.from_numpy(rng.standard_normal((n, e)).astype(np.float32)).to(DEV)
    x = torch.from_numpy(rng.standard_normal((n, d)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    return logits, x


def _compare(logits, x, xs, k, g, sort, cutoff=256, renorm=True):
    ref = moe.moe_route_dispatch(logits, x, k, g, renorm, sort, cutoff, x_scales=xs)
    got = moe.moe_route_dispatch_noalloc(logits, x, k, g, renorm, sort, cutoff, x_scales=xs)
    torch.cuda.synchronize()
    assert got[2].sorted == ref[2].sorted
    assert np.array_equal(_bits(got[0]), _bits(ref[0])), "topk_idx"
    assert np.array_equal(_bits(got[1]), _bits(ref[1])), "topk_w"
    for f in FIELDS:
        a, b = _bits(getattr(got[2], f)), _bits(getattr(ref[2], f))
        assert (a is None) == (b is None), f
        if a is not None:
            assert np.array_equal(a, b), f


@pytest.mark.parametrize("first,second", [
    (("prefill", None, 1), ("decode", None, 0)),          # sorted 4096 tokens, then the identity layout
    (("segment", None, 1), ("segment", 100, 0)),          # fp8 + scales, G = 8, both sort modes
    (("mixtral", None, -1), ("tiny", None, -1)),          # auto mode: sorted, then unsorted
])
def test_noalloc_matches_workspace_call(first, second):
    for name, n, sort in (first, second):
        cfg, logits, x, xs = _inputs(name, n)
        _compare(logits, x, xs, cfg.top_k, cfg.n_segments, sort, cfg.sort_cutoff, cfg.renormalize)


def test_noalloc_at_the_scratch_limit_then_smaller():
    """E = 1024 with 32768 tokens x top-8 needs exactly the whole array (256
    chunk histograms of 4 KB plus 256 bytes); then a small call on top."""
    n, e, k = 32768, 1024, 8
    assert moe.moe_route_dispatch_workspace_bytes(n, e, k, 1) == moe.MOE_NOALLOC_SCRATCH_BYTES
    logits, x = _random_inputs(n, e, 64, 1)
    _compare(logits, x, None, k, 1, 1)
    logits, x = _random_inputs(300, e, 64, 2)
    _compare(logits, x, None, k, 4, 1)
    _compare(logits, x, None, k, 4, 0)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    n, e, k = 1 << 16, 1024, 8
    logits = torch.zeros((n, e), dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError, match="static array"):
        moe.moe_route_dispatch_noalloc(logits, None, k, 1, sort=1)


@pytest.mark.parametrize("name,sort", [("prefill", 1), ("decode", 0), ("segment", 1)])
def test_noalloc_under_graph_capture(name, sort):
    """The callers this entry point is for: captured in a HIP graph with its
    outputs preallocated (nothing is allocated during capture), replayed four
    times.  Before each replay every output is clobbered and an eager call of
    the same entry point on other inputs runs on the same static scratch; each
    replay must reproduce the eager result bit for bit."""
    cfg, logits, x, xs = _inputs(name)
    k, g = cfg.top_k, cfg.n_segments
    idx, w, res = moe.moe_route_dispatch_noalloc(logits, x, k, g, cfg.renormalize, sort, cfg.sort_cutoff,
                                                 x_scales=xs)
    torch.cuda.synchronize()
    outputs = [idx, w] + [getattr(res, f) for f in FIELDS if getattr(res, f) is not None]
    eager = [_bits(t).copy() for t in outputs]
    other_logits = torch.flip(logits, dims=[0]).contiguous()      # a different routing

    def step():
        moe.moe_route_dispatch_noalloc(logits, x, k, g, cfg.renormalize, sort, cfg.sort_cutoff,
                                       x_scales=xs, topk_idx=idx, topk_w=w, out=res)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in outputs:
            t.zero_()
        moe.moe_route_dispatch_noalloc(other_logits, x, k, g, cfg.renormalize, sort, cfg.sort_cutoff,
                                       x_scales=xs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(outputs):
            assert np.array_equal(_bits(t), eager[i]), (rep, i)
