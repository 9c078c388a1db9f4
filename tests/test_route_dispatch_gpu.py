"""moe_route_dispatch equals moe_route_topk followed by moe_dispatch, bit for
bit, and both equal the oracle."""
import os

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


@pytest.mark.parametrize("n,e,k,g,sort", [
    (8192, 8, 2, 1, 1),        # the Mixtral-like shape
    (8192, 8, 2, 4, 0),        # segments (unsorted)
    (2049, 16, 4, 4, 1), (2049, 16, 4, 2, 0),   # ragged last routing workgroup
    (32768, 4, 1, 1, 1), (32769, 4, 1, 1, 1),
    (4097, 2, 2, 2, 1), (5000, 16, 8, 16, 1), (8192, 16, 1, 1, 1),
    (6000, 8, 3, 1, 1),        # k = 3
    (3000, 12, 2, 3, 1),       # E = 12
])
def test_few_experts(n, e, k, g, sort):
    """At most 16 experts above the one-workgroup size, ragged token counts,
    k = 3 and non-power-of-two E; skewed logits make a few experts popular."""
    rng = np.random.default_rng(n * 7 + e + k)
    logits = rng.standard_normal((n, e)).astype(np.float32)
    logits[:, 0] += 1.5
    x = rng.integers(0, 2**16, (n, 40), dtype=np.uint16)
    _compare(logits, x, k, g, sort)


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


@pytest.mark.parametrize("n,e,k,g,sort,dtype,d", [
    (4096, 256, 8, 1, 1, "bf16", 7168),    # prefill shape
    (8192, 8, 2, 1, 1, "bf16", 4096),      # Mixtral-like shape
    (1024, 256, 8, 8, 0, "f8", 7168),      # segment-major fp8 rows and block scales
    (3001, 256, 8, 4, 1, "f32", 100),      # ragged last chunk, 400-byte rows
    (2100, 100, 9, 10, 0, "bf16", 8),      # one 16-byte vector per row
    (4097, 584, 1, 1, 1, "bf16", 64),      # the largest E whose rank LDS fits 16 KB
    (4097, 585, 1, 1, 1, "bf16", 64),      # one expert more: ranks and copy in separate launches
    (128, 256, 8, 1, 0, "bf16", 7168),     # identity layout: routing and row copy in one launch
    (300, 64, 4, 2, 1, "bf16", 64),        # 1200 pairs: the one-workgroup metadata path
])
def test_route_dispatch_in_validate_mode(n, e, k, g, sort, dtype, d):
    """moe_route_dispatch with validate mode on, over its launch forms: positions
    and row copy in one launch (16-byte rows, above 4096 pairs, outside the
    identity layout, rank LDS within 16 KB), in separate launches (E = 585),
    the identity layout's routing-and-copy launch and the one-workgroup
    metadata path.  The call waits and fails if any copy wave gave up waiting
    for its positions; every map and row is compared with the oracle's
    routing and dispatch."""
    rng = np.random.default_rng(n + e + d)
    logits = rng.standard_normal((n, e)).astype(np.float32)
    xs = None
    if dtype == "f8":
        x = rng.integers(0, 256, (n, d), dtype=np.uint8)
        x[(x & 0x7F) == 0x7F] = 0
        xs = rng.uniform(0.5, 2.0, (n, d // 128)).astype(np.float32)
    elif dtype == "bf16":
        x = rng.integers(0, 2**16, (n, d), dtype=np.uint16)
    else:
        x = rng.standard_normal((n, d)).astype(np.float32)
    os.environ["MOE_DC_VALIDATE"] = "1"
    try:
        idx, _, res = moe.moe_route_dispatch(to_dev(logits), to_dev(x), k, g, True, sort,
                                             x_scales=None if xs is None else to_dev(xs))
    finally:
        del os.environ["MOE_DC_VALIDATE"]
    oi, _ = oracle_route(logits, k, True)
    assert np.array_equal(to_np(idx), oi)
    ref = od.dispatch(oi, e, g, bool(sort), x=x, x_scales=xs)
    for name in MAPS:
        assert np.array_equal(to_np(getattr(res, name)), ref[name]), name
    assert np.array_equal(to_np(res.rows).view(np.uint8), ref["rows"].view(np.uint8))
    if xs is not None:
        assert np.array_equal(to_np(res.row_scales), ref["row_scales"])


def test_rank_and_copy_give_up_path_is_reported():
    """moe_route_dispatch's shared rank + copy launch: with the copy waves'
    poll limit forced to 0 from the host (MOE_DC_SPIN_LIMIT, a test hook),
    waves that find their positions not yet published give up at once, the
    launch still ends normally, those rows are skipped and validate mode
    reports it (at the prefill size this is all but certain; a call where no
    wave had to wait must then be exact).  The next call, with the default
    limit, is exact."""
    cfg = CONFIGS["prefill"]
    inp = make_inputs(cfg)
    logits = to_dev(inp["logits"])
    x = to_dev(inp["x"])
    oi, _ = oracle_route(inp["logits"], cfg.top_k, cfg.renormalize)
    ref = od.dispatch(oi, cfg.n_experts, 1, True)
    rng = np.random.default_rng(5)
    sample = rng.integers(0, cfg.n_tokens * cfg.top_k, 4000)

    def exact(res):
        for name in MAPS:
            assert np.array_equal(to_np(getattr(res, name)), ref[name]), name
        rows = res.rows[torch.from_numpy(sample).to(DEV)]
        assert np.array_equal(to_np(rows), inp["x"][ref["src_pair"][sample] // cfg.top_k])

    os.environ["MOE_DC_VALIDATE"] = "1"
    try:
        os.environ["MOE_DC_SPIN_LIMIT"] = "0"
        try:
            _, _, res = moe.moe_route_dispatch(logits, x, cfg.top_k, 1, cfg.renormalize, 1)
            exact(res)
        except moe.MoeError as err:
            assert "gave up" in str(err)
        finally:
            del os.environ["MOE_DC_SPIN_LIMIT"]
        _, _, res = moe.moe_route_dispatch(logits, x, cfg.top_k, 1, cfg.renormalize, 1)
        exact(res)
    finally:
        del os.environ["MOE_DC_VALIDATE"]
