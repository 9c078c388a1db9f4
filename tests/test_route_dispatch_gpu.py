"""moe_route_dispatch equals moe_route_topk followed by moe_dispatch, bit for
bit, and both equal the oracle."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from oracle import dispatch as od
from oracle.route import route_topk as oracle_route
from tests.gpu_util import DEV, to_dev, to_np
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu

MAPS = ("expert_counts", "expert_offsets", "segment_offsets", "src_pair", "dst_pos", "row_expert")


def _compare(logits, x, k, g, sort, x_scales=None, renorm=True, cutoff=256):
    e = logits.shape[1]
    xd = None if x is None else to_dev(x)
    xs = None if x_scales is None else to_dev(x_scales)
    idx_f, w_f, res_f = moe.moe_route_dispatch(to_dev(logits), xd, k, g, renorm, sort, cutoff, x_scales=xs)
    idx_s, w_s = moe.moe_route_topk(to_dev(logits), k, renorm)
    res_s = moe.moe_dispatch(xd, idx_s, e, g, sort=sort, sort_cutoff=cutoff, x_scales=xs)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(idx_f), to_np(idx_s))
    assert np.array_equal(to_np(w_f).view(np.uint32), to_np(w_s).view(np.uint32))
    assert res_f.sorted == res_s.sorted
    for name in MAPS:
        assert np.array_equal(to_np(getattr(res_f, name)), to_np(getattr(res_s, name))), name
    if x is not None:
        assert np.array_equal(to_np(res_f.rows).view(np.uint8), to_np(res_s.rows).view(np.uint8))
    if x_scales is not None:
        assert np.array_equal(to_np(res_f.row_scales), to_np(res_s.row_scales))
    if logits.shape[0] == 0:
        return
    oi, _ = oracle_route(logits, k, renorm)
    assert np.array_equal(to_np(idx_f), oi)
    ref = od.dispatch(oi, e, g, res_f.sorted, x=x)
    for name in MAPS:
        assert np.array_equal(to_np(getattr(res_f, name)), ref[name]), name
    if x is not None:
        assert np.array_equal(to_np(res_f.rows).view(np.uint8), ref["rows"].view(np.uint8))


@pytest.mark.parametrize("sort,g", [(1, 1), (0, 1), (0, 8), (1, 8)])
def test_prefill_shape(sort, g):
    cfg = CONFIGS["prefill"]
    inp = make_inputs(cfg)
    _compare(inp["logits"], inp["x"], cfg.top_k, g, sort)


@pytest.mark.parametrize("n,e,k,g,sort", [
    (3001, 256, 8, 4, 1),      # ragged last 64-token chunk
    (20000, 64, 4, 1, 1),      # 79 counting chunks
    (9000, 8, 1, 2, 1),        # k = 1 above the one-workgroup size
    (9000, 8, 2, 1, 1),        # k = 2 above the one-workgroup size
    (500, 1024, 8, 16, 1),     # E = 1024 (16 logits per lane)
    (500, 1024, 8, 16, 0),
    (65, 512, 64, 2, 1),       # k = 64
    (2100, 100, 9, 10, 0),
    (10, 16, 4, 4, 1),         # one-workgroup path
    (0, 16, 4, 4, 1),
    (128, 256, 8, 1, 0),       # identity layout: routing and row copy in one launch
    (37, 64, 3, 1, 0),
    (1, 16, 16, 1, 0),
    (5000, 1024, 8, 1, 0),     # identity layout, count + rank maps, 16 logits per lane
    (50, 8, 1, 1, 0),          # identity layout, k = 1
    (9, 1, 1, 1, 0),           # one expert
])
def test_shapes(n, e, k, g, sort):
    rng = np.random.default_rng(n + e + k)
    logits = rng.standard_normal((n, e)).astype(np.float32)
    x = rng.integers(0, 2**16, (n, 24), dtype=np.uint16)
    _compare(logits, x, k, g, sort)
    _compare(logits, None, k, g, sort, renorm=False)


@pytest.mark.parametrize("cols", [5, 12, 1000])   # 10-, 24- and 2000-byte rows: not 16-byte multiples
def test_identity_layout_narrow_rows(cols):
    rng = np.random.default_rng(cols)
    logits = rng.standard_normal((70, 32)).astype(np.float32)
    x = rng.integers(0, 2**16, (70, cols), dtype=np.uint16)
    _compare(logits, x, 4, 1, 0)


def test_fp8_segment_workload_and_auto_mode():
    cfg = CONFIGS["segment"]
    inp = make_inputs(cfg)
    for sort in (0, 1, -1):
        _compare(inp["logits"], inp["x"], cfg.top_k, cfg.n_segments, sort, x_scales=inp["x_scales"],
                 cutoff=512)
