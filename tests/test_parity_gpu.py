"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer outputs (indices, counts, offsets, maps, dispatched rows) must match
bit for bit; floating-point outputs within the tolerances in gpu_util.
"""
import os

import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from oracle import codecs, dispatch as od
from oracle.experts import dequant_rows
from oracle.route import route_topk as oracle_route
from tests.gpu_util import (DEV, as_f32, check_combine, check_weights, combine_check_all_tokens,
                            combine_reference, to_dev, to_np)
from workloads import CONFIGS, alternating_sort, make_inputs

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


def _route_check(logits: np.ndarray, k: int, renorm: bool = True):
    idx, w = moe.moe_route_topk(to_dev(logits), k, renorm)
    _sync()
    oi, ow = oracle_route(logits, k, renorm)
    gi, gw = to_np(idx), to_np(w)
    assert np.array_equal(gi, oi), f"indices differ in {np.sum(gi != oi)} places"
    check_weights(gw, ow, f"N={logits.shape[0]} E={logits.shape[1]} k={k} renorm={renorm}")
    return idx, w


def _dispatch_check(idx_dev, n_experts, n_segments, sort, x=None, x_scales=None, cutoff=256,
                    rows_sample=None):
    res = moe.moe_dispatch(None if x is None else to_dev(x), idx_dev, n_experts, n_segments,
                           sort=sort, sort_cutoff=cutoff,
                           x_scales=None if x_scales is None else to_dev(x_scales))
    _sync()
    idx = to_np(idx_dev)
    n = idx.shape[0]
    assert res.sorted == od.resolve_sorted(sort, n, cutoff)
    ref = od.dispatch(idx, n_experts, n_segments, res.sorted)
    for name in ("expert_counts", "expert_offsets", "segment_offsets", "src_pair", "dst_pos",
                 "row_expert"):
        got = to_np(getattr(res, name))
        assert np.array_equal(got, ref[name]), f"{name} differs ({np.sum(got != ref[name])} entries)"
    if x is not None:
        rows = to_np(res.rows)
        k = idx.shape[1]
        if rows_sample is None:
            expect = od.gather_rows(x, ref["src_pair"], k)
            assert np.array_equal(rows.view(np.uint8), expect.view(np.uint8)), "rows differ"
        else:
            ps = rows_sample
            expect = np.asarray(x)[ref["src_pair"][ps] // k]
            assert np.array_equal(rows[ps].view(np.uint8), expect.view(np.uint8)), "sampled rows differ"
        if x_scales is not None:
            assert np.array_equal(to_np(res.row_scales), od.gather_rows(x_scales, ref["src_pair"], k))
    return res


# ----------------------------------------------------------------- routing

@pytest.mark.parametrize("name", list(CONFIGS))
@pytest.mark.parametrize("renorm", [True, False])
def test_route_full_size(name, renorm):
    """Every workload's logits, with the weights renormalised over the top k
    (the workloads' setting) and as the full softmax (weights ~1/E, where an
    absolute tolerance would hide relative errors)."""
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    _route_check(inp["logits"], cfg.top_k, renorm)


@pytest.mark.parametrize("n,e,k", [(1, 1, 1), (7, 5, 3), (33, 64, 64), (100, 65, 8),
                                   (64, 129, 2), (50, 1000, 32), (300, 1024, 8), (17, 256, 1),
                                   (5, 256, 16), (3, 16, 16), (31, 255, 9), (1, 256, 8)])
@pytest.mark.parametrize("renorm", [True, False])
def test_route_shapes(n, e, k, renorm):
    rng = np.random.default_rng(n * 1000 + e)
    _route_check(rng.standard_normal((n, e)).astype(np.float32), k, renorm)


def test_route_ties_and_signed_zero():
    rng = np.random.default_rng(9)
    pool = np.array([-1.0, -0.0, 0.0, 0.5, 2.0], dtype=np.float32)
    logits = pool[rng.integers(0, pool.size, (500, 96))]
    _route_check(logits, 8)
    _route_check(np.zeros((4, 256), np.float32), 8)          # all equal: 0..7, w = 1/8
    _route_check(-np.arange(300, dtype=np.float32)[None].repeat(3, 0), 16)
    big = rng.standard_normal((64, 256)).astype(np.float32) * 80   # large spread in exp()
    _route_check(big, 8)
    _route_check(big, 8, renorm=False)
    # differences l_j - l_0 of up to ~80 whose fp32 subtraction rounds: the weight
    # must come from the exact difference (exp(l_j - l_0) is down to ~1e-35 here)
    near = (rng.standard_normal((256, 64)) * 20).astype(np.float32)
    near[:, 0] = 40.0 + rng.uniform(0, 1, 256).astype(np.float32)
    _route_check(near, 16)
    _route_check(near, 64, renorm=False)
    wide = (rng.standard_normal((128, 1024)) * 30).astype(np.float32)
    _route_check(wide, 32)
    _route_check(wide, 8, renorm=False)


def test_route_empty():
    idx, w = moe.moe_route_topk(torch.empty((0, 8), dtype=torch.float32, device=DEV), 2)
    assert idx.shape == (0, 2)


# ----------------------------------------------------------------- dispatch

@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mixtral", "segment"])
def test_dispatch_full_size(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    idx, _ = moe.moe_route_topk(to_dev(inp["logits"]), cfg.top_k, cfg.renormalize)
    sorts = [0, 1] if cfg.sort == "alternate" else [cfg.sort]
    for s in sorts:
        _dispatch_check(idx, cfg.n_experts, cfg.n_segments, s, x=inp["x"], x_scales=inp["x_scales"],
                        cutoff=cfg.sort_cutoff)


@pytest.mark.parametrize("n,e,k,g", [
    (1, 8, 2, 1), (3, 8, 8, 2), (129, 16, 4, 4), (512, 256, 8, 8),      # one-workgroup path (NK <= 4096)
    (513, 256, 8, 8), (2047, 256, 8, 8), (3000, 64, 8, 4), (2049, 32, 8, 1),   # multi-block path
    (100, 512, 4, 8), (300, 1024, 8, 1024), (5000, 1024, 1, 16), (64, 1000, 32, 8),
])
@pytest.mark.parametrize("sort", [0, 1])
def test_dispatch_shapes(n, e, k, g, sort):
    rng = np.random.default_rng(n + e + k)
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    x = rng.integers(0, 2**16, (n, 40), dtype=np.uint16)             # 80-byte rows
    _dispatch_check(to_dev(idx), e, g, sort, x=x)


@pytest.mark.parametrize("n,e,k,g", [(500, 8, 4, 2), (20000, 16, 2, 4)])
def test_dispatch_duplicate_ids_and_skew(n, e, k, g):
    # ids repeated inside a token and most pairs on one expert
    rng = np.random.default_rng(4)
    idx = np.where(rng.uniform(size=(n, k)) < 0.8, 3, rng.integers(0, e, (n, k))).astype(np.int32)
    for sort in (0, 1):
        _dispatch_check(to_dev(idx), e, g, sort, x=rng.standard_normal((n, 8)).astype(np.float32))


@pytest.mark.parametrize("n,e,k,g,sort", [
    (2049, 16, 2, 1, 1), (8192, 8, 2, 1, 1), (4097, 8, 1, 8, 1), (1025, 256, 8, 8, 0),
    (2048, 1024, 8, 16, 0), (16384, 4, 1, 2, 0), (8000, 16, 2, 4, 1), (8192, 8, 2, 1, 0),
])
@pytest.mark.parametrize("skew", [False, True])
def test_dispatch_few_buckets(n, e, k, g, sort, skew):
    """4K < N*k <= 16K pairs with at most 16 buckets (experts when sorted,
    segments when not), where many pairs share each bucket's counters.
    Uniform and skewed routing (80% of the pairs on one expert)."""
    rng = np.random.default_rng(n + e + g + sort)
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    if skew:
        idx = np.where(rng.uniform(size=(n, k)) < 0.8, 3 % e, idx).astype(np.int32)
    x = rng.integers(0, 2**16, (n, 24), dtype=np.uint16)
    _dispatch_check(to_dev(idx), e, g, sort, x=x)


@pytest.mark.parametrize("row_elems,dtype", [(3, np.uint16), (5, np.uint16), (6, np.uint16),
                                             (4, np.uint16), (7, np.float32), (1, np.float32),
                                             (2, np.float32)])
def test_dispatch_narrow_rows(row_elems, dtype):
    # row sizes of 6, 10, 12, 8, 28, 4 and 8 bytes take the 2-, 4- and 8-byte copy paths
    rng = np.random.default_rng(row_elems)
    n, e, k = 77, 16, 3
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    if dtype == np.float32:
        x = rng.standard_normal((n, row_elems)).astype(np.float32)
    else:
        x = rng.integers(0, 2**16, (n, row_elems), dtype=np.uint16)
    for sort in (0, 1):
        _dispatch_check(to_dev(idx), e, 1, sort, x=x)


def test_dispatch_auto_mode_and_cutoffs():
    rng = np.random.default_rng(8)
    for n, cutoff in ((256, 256), (257, 256), (5, 0), (5, 4), (1, 1)):
        idx = np.stack([rng.permutation(32)[:4] for _ in range(n)]).astype(np.int32)
        _dispatch_check(to_dev(idx), 32, 2, -1, cutoff=cutoff,
                        x=rng.standard_normal((n, 16)).astype(np.float32))


def test_dispatch_empty():
    idx = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    res = moe.moe_dispatch(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), idx, 16, 4, sort=1)
    _sync()
    assert (to_np(res.expert_counts) == 0).all()
    assert (to_np(res.expert_offsets) == 0).all() and res.expert_offsets.numel() == 17
    assert (to_np(res.segment_offsets) == 0).all() and res.segment_offsets.numel() == 5


def test_dispatch_reuses_buffers_across_modes():
    # the segment-major workload toggles the sort flag on consecutive calls
    cfg = CONFIGS["segment"]
    inp = make_inputs(cfg)
    idx, _ = moe.moe_route_topk(to_dev(inp["logits"]), cfg.top_k)
    out = None
    ws = torch.empty(moe.moe_dispatch_workspace_bytes(cfg.n_tokens, cfg.n_experts, cfg.top_k,
                                                      cfg.n_segments), dtype=torch.uint8, device=DEV)
    x, xs = to_dev(inp["x"]), to_dev(inp["x_scales"])
    for call in range(4):
        s = alternating_sort(call)
        out = moe.moe_dispatch(x, idx, cfg.n_experts, cfg.n_segments, sort=s, x_scales=xs,
                               workspace=ws, out=out)
        _sync()
        ref = od.dispatch(to_np(idx), cfg.n_experts, cfg.n_segments, bool(s), x=inp["x"],
                          x_scales=inp["x_scales"])
        assert out.sorted == bool(s)
        for name in ("src_pair", "dst_pos", "row_expert", "expert_offsets", "segment_offsets"):
            assert np.array_equal(to_np(getattr(out, name)), ref[name]), (call, name)
        assert np.array_equal(to_np(out.rows), ref["rows"])
        assert np.array_equal(to_np(out.row_scales), ref["row_scales"])


def test_dispatch_validate_mode_reports_bad_ids_few_buckets():
    """Out-of-range ids are flagged on the multi-workgroup counting path too."""
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 8, (6000, 2)).astype(np.int32)
    idx[1234, 1] = 8
    os.environ["MOE_DC_VALIDATE"] = "1"
    try:
        with pytest.raises(moe.MoeError, match="outside"):
            moe.moe_dispatch(None, to_dev(idx), 8, 1, sort=1)
        idx[1234, 1] = 7
        moe.moe_dispatch(None, to_dev(idx), 8, 1, sort=1)
    finally:
        del os.environ["MOE_DC_VALIDATE"]


def test_dispatch_validate_mode_reports_bad_ids():
    idx = torch.tensor([[0, 1], [2, 9]], dtype=torch.int32, device=DEV)
    os.environ["MOE_DC_VALIDATE"] = "1"
    try:
        with pytest.raises(moe.MoeError, match="outside"):
            moe.moe_dispatch(torch.zeros((2, 16), dtype=torch.bfloat16, device=DEV), idx, 8, 1, sort=1)
        good = torch.tensor([[0, 1], [2, 7]], dtype=torch.int32, device=DEV)
        moe.moe_dispatch(torch.zeros((2, 16), dtype=torch.bfloat16, device=DEV), good, 8, 1, sort=1)
    finally:
        del os.environ["MOE_DC_VALIDATE"]


@pytest.mark.parametrize("n,e,k,g,sort,dtype,d", [
    (5000, 256, 8, 1, 1, "bf16", 64),      # sorted, 40000 pairs
    (3000, 7, 3, 7, 0, "f32", 12),         # segments (unsorted), 48-byte rows
    (2049, 64, 2, 1, 1, "bf16", 8),        # 4098 pairs: just above the one-workgroup path
    (2048, 64, 4, 4, 1, "f8", 512),        # fp8 rows with 16-byte scale rows: both in the launch
    (2048, 64, 4, 4, 1, "f8", 256),        # 8-byte scale rows: separate row copies
    (3000, 16, 2, 1, 1, "bf16", 100),      # 200-byte rows (not 16-byte): separate row copy
])
def test_rank_and_copy_launch_in_validate_mode(n, e, k, g, sort, dtype, d):
    """Ranks and row copy sharing one launch (16-byte rows, above 4096 pairs,
    outside the identity layout), with validate mode on: the call waits and
    fails if any copy wave gave up waiting for its positions; every map and
    row is compared with the oracle."""
    rng = np.random.default_rng(n + e + d)
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
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
        res = moe.moe_dispatch(to_dev(x), to_dev(idx), e, g, sort=sort,
                               x_scales=None if xs is None else to_dev(xs))
    finally:
        del os.environ["MOE_DC_VALIDATE"]
    ref = od.dispatch(idx, e, g, bool(sort), x=x, x_scales=xs)
    for name in ("expert_counts", "expert_offsets", "segment_offsets", "src_pair", "dst_pos", "row_expert"):
        assert np.array_equal(to_np(getattr(res, name)), ref[name]), name
    assert np.array_equal(to_np(res.rows).view(np.uint8), ref["rows"].view(np.uint8))
    if xs is not None:
        assert np.array_equal(to_np(res.row_scales), ref["row_scales"])


def test_rank_and_copy_give_up_path_is_reported():
    """The copy waves of the shared rank + copy launch wait a bounded number of
    polls for their positions.  With the limit forced to 0 from the host
    (MOE_DC_SPIN_LIMIT, a test hook), waves that find their positions not yet
    published give up at once: the launch still ends normally, those rows are
    skipped, and validate mode reports it (at the prefill size the first copy
    waves poll long before the rank workgroups finish, so this is all but
    certain; a call where no wave had to wait must then be exact).  The next
    call, with the default limit, is exact again."""
    cfg = CONFIGS["prefill"]
    inp = make_inputs(cfg)
    idx, _ = moe.moe_route_topk(to_dev(inp["logits"]), cfg.top_k)
    x = to_dev(inp["x"])
    ref = od.dispatch(to_np(idx), cfg.n_experts, 1, True)
    rng = np.random.default_rng(3)
    sample = rng.integers(0, cfg.n_tokens * cfg.top_k, 4000)
    xh = inp["x"]

    def exact(res):
        for name in ("expert_counts", "expert_offsets", "src_pair", "dst_pos", "row_expert"):
            assert np.array_equal(to_np(getattr(res, name)), ref[name]), name
        rows = res.rows[torch.from_numpy(sample).to(DEV)]
        assert np.array_equal(to_np(rows), xh[ref["src_pair"][sample] // cfg.top_k])

    os.environ["MOE_DC_VALIDATE"] = "1"
    try:
        os.environ["MOE_DC_SPIN_LIMIT"] = "0"
        try:
            res = moe.moe_dispatch(x, idx, cfg.n_experts, 1, sort=1)
            exact(res)
        except moe.MoeError as err:
            assert "gave up" in str(err)
        finally:
            del os.environ["MOE_DC_SPIN_LIMIT"]
        exact(moe.moe_dispatch(x, idx, cfg.n_experts, 1, sort=1))
    finally:
        del os.environ["MOE_DC_VALIDATE"]


# ----------------------------------------------------------------- combine

def _combine_case(x_np, idx_dev, w_dev, e, g, sort, out_bf16):
    """Dispatch, identity experts, combine; every token checked (in chunks)."""
    res = moe.moe_dispatch(to_dev(x_np), idx_dev, e, g, sort=sort)
    y = res.rows                                   # identity experts
    out = moe.moe_combine(y, res.dst_pos, w_dev, out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    _sync()
    combine_check_all_tokens(out, y, res.dst_pos, w_dev, w_dev.shape[1], out_bf16, what=f"sort={sort}")
    return out


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "segment"])
def test_combine_identity_experts_full_size(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    idx, w = moe.moe_route_topk(to_dev(inp["logits"]), cfg.top_k, cfg.renormalize)
    sort = 1 if cfg.sort == "alternate" else cfg.sort
    if cfg.dtype == "f8":
        res = moe.moe_dispatch(to_dev(inp["x"]), idx, cfg.n_experts, cfg.n_segments, sort=sort,
                               x_scales=to_dev(inp["x_scales"]))
        y = moe.moe_dequant_rows(res.rows, res.row_scales)
        _sync()
        y_ref = dequant_rows(to_np(res.rows), to_np(res.row_scales))
        assert np.array_equal(to_np(y), y_ref), "dequantised rows differ"
        out = moe.moe_combine(y, res.dst_pos, w)
        _sync()
        exact, mag = combine_reference(as_f32(y_ref), to_np(res.dst_pos), to_np(w), cfg.top_k)
        check_combine(to_np(out), exact, mag, True, what=name)
        return
    out_bf16 = cfg.dtype == "bf16"
    out = _combine_case(inp["x"], idx, w, cfg.n_experts, cfg.n_segments, sort, out_bf16)
    # identity experts with weights summing to one reproduce the input
    x = as_f32(inp["x"]).astype(np.float64)
    got = as_f32(to_np(out)).astype(np.float64)
    # bf16: the fp32 chain is within ~2k fp32 ulps of x, far inside half a bf16 ulp;
    # fp32: k roundings of the weights plus k roundings of the chain
    rel = 2.0 ** -8 if out_bf16 else (2 * cfg.top_k + 2) * 2.0 ** -24
    assert np.all(np.abs(got - x) <= rel * np.abs(x) + 1e-30)


@pytest.mark.parametrize("n,e,k,d", [(1, 4, 1, 8), (37, 16, 3, 24), (200, 64, 8, 136),
                                     (90, 32, 5, 36), (64, 256, 32, 512), (333, 8, 2, 7)])
@pytest.mark.parametrize("y_bf16,out_bf16", [(False, False), (True, True), (True, False), (False, True)])
def test_combine_random_experts(n, e, k, d, y_bf16, out_bf16):
    rng = np.random.default_rng(n * d + k)
    nk = n * k
    y = rng.standard_normal((nk, d)).astype(np.float32)
    if y_bf16:
        y = codecs.f32_to_bf16_bits(y)
    dst = rng.permutation(nk).astype(np.int32)
    w = rng.uniform(-1, 1, (n, k)).astype(np.float32)                 # signs mix: cancellation
    out = moe.moe_combine(to_dev(y), to_dev(dst), to_dev(w),
                          out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    _sync()
    exact, mag = combine_reference(as_f32(y), dst, w, k)
    check_combine(to_np(out), exact, mag, out_bf16, what=f"{n},{e},{k},{d}")


def test_combine_sorted_equals_unsorted_bitwise():
    for name in ("decode", "segment", "tiny"):
        cfg = CONFIGS[name]
        inp = make_inputs(cfg)
        x = inp["x"] if cfg.dtype != "f8" else codecs.f32_to_bf16_bits(
            codecs.fp8_bits_to_f64(inp["x"]).astype(np.float32))
        idx, w = moe.moe_route_topk(to_dev(inp["logits"]), cfg.top_k)
        outs = []
        for sort, g in ((0, 1), (1, 1), (0, cfg.n_segments), (1, cfg.n_segments), (0, 2), (1, 2)):
            res = moe.moe_dispatch(to_dev(x), idx, cfg.n_experts, g, sort=sort)
            outs.append(to_np(moe.moe_combine(res.rows, res.dst_pos, w)))
        _sync()
        for o in outs[1:]:
            assert np.array_equal(o.view(np.uint8), outs[0].view(np.uint8)), name


def test_round_trip_one_hot_is_exact():
    # dispatch then combine with one-hot weights returns every token's row
    rng = np.random.default_rng(12)
    for dtype, (n, e, k, d) in (("bf16", (300, 64, 8, 256)), ("f32", (77, 8, 2, 64))):
        xf = rng.standard_normal((n, d)).astype(np.float32)
        x = codecs.f32_to_bf16_bits(xf) if dtype == "bf16" else xf
        idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
        for sort in (0, 1):
            res = moe.moe_dispatch(to_dev(x), to_dev(idx), e, 4 if e % 4 == 0 else 1, sort=sort)
            for hot in (0, k - 1):
                w = np.zeros((n, k), np.float32)
                w[:, hot] = 1.0
                out = to_np(moe.moe_combine(res.rows, res.dst_pos, to_dev(w)))
                assert np.array_equal(out.view(np.uint8), x.view(np.uint8)), (dtype, sort, hot)


def test_combine_is_deterministic_and_weight_scaling_exact():
    cfg = CONFIGS["prefill"].with_tokens(1024)
    inp = make_inputs(cfg)
    idx, w = moe.moe_route_topk(to_dev(inp["logits"]), cfg.top_k)
    res = moe.moe_dispatch(to_dev(inp["x"]), idx, cfg.n_experts, 1, sort=1)
    a = to_np(moe.moe_combine(res.rows, res.dst_pos, w, out_dtype=torch.float32))
    b = to_np(moe.moe_combine(res.rows, res.dst_pos, w, out_dtype=torch.float32))
    c = to_np(moe.moe_combine(res.rows, res.dst_pos, w * 2, out_dtype=torch.float32))
    assert np.array_equal(a, b)
    assert np.array_equal(c, 2 * a)


def test_combine_skips_out_of_range_positions():
    y = torch.ones((4, 16), dtype=torch.float32, device=DEV)
    dst = torch.tensor([0, -1, 7, 3], dtype=torch.int32, device=DEV)
    w = torch.full((2, 2), 0.5, dtype=torch.float32, device=DEV)
    out = to_np(moe.moe_combine(y, dst, w))
    assert (out == 0.5).all()


# ----------------------------------------------------------------- experts

def test_dequant_rows_bit_exact():
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 256, (300, 384), dtype=np.uint8)
    rows[(rows & 0x7F) == 0x7F] = 0x41                 # no NaN codes
    scales = np.exp(rng.uniform(-12, 3, (300, 3))).astype(np.float32)
    scales[0, 0] = 2.0 ** -140                         # products in the subnormal range
    y = moe.moe_dequant_rows(to_dev(rows), to_dev(scales))
    _sync()
    assert np.array_equal(to_np(y), dequant_rows(rows, scales))


# ----------------------------------------------------------------- graph capture

def test_path_in_hip_graph_matches_eager_every_replay():
    """route -> dispatch -> scatter -> combine captured in one graph; every
    replay (with eager work and syncs in between) equals the eager result."""
    cfg = CONFIGS["decode"]
    inp = make_inputs(cfg)
    logits, x = to_dev(inp["logits"]), to_dev(inp["x"])
    n, k = cfg.n_tokens, cfg.top_k
    idx = torch.empty((n, k), dtype=torch.int32, device=DEV)
    w = torch.empty((n, k), dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.moe_dispatch_workspace_bytes(n, cfg.n_experts, k, 1), dtype=torch.uint8, device=DEV)
    res = moe.moe_dispatch(None, idx.zero_(), cfg.n_experts, 1, sort=1, workspace=ws)
    rows = torch.empty((n * k, cfg.hidden), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((n, cfg.hidden), dtype=torch.bfloat16, device=DEV)

    def step(sort):
        moe.moe_route_topk(logits, k, topk_idx=idx, topk_w=w)
        moe.moe_dispatch(None, idx, cfg.n_experts, 1, sort=sort, workspace=ws, out=res)
        moe.moe_scatter_rows(x, res.dst_pos, k, rows=rows)
        moe.moe_combine(rows, res.dst_pos, w, out=out)

    for sort in (0, 1):
        step(sort)
        _sync()
        eager = (to_np(out).copy(), to_np(res.dst_pos).copy(), to_np(rows).copy())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(sort)
        for rep in range(4):
            out.zero_()
            rows.zero_()
            res.dst_pos.fill_(-7)
            _sync()
            g.replay()
            _sync()
            assert np.array_equal(to_np(out), eager[0]), (sort, rep)
            assert np.array_equal(to_np(res.dst_pos), eager[1]), (sort, rep)
            assert np.array_equal(to_np(rows), eager[2]), (sort, rep)


# ----------------------------------------------------------------- row copies on their own

@pytest.mark.parametrize("row_elems,np_dtype", [(7168, np.uint16), (40, np.uint16), (3, np.uint16),
                                                (64, np.float32), (5, np.float32)])
@pytest.mark.parametrize("sort", [0, 1])
def test_scatter_and_gather_rows_forms(row_elems, np_dtype, sort):
    rng = np.random.default_rng(row_elems + sort)
    n, e, k, g = 300, 64, 8, 4
    idx = np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)
    x = (rng.integers(0, 2**16, (n, row_elems), dtype=np.uint16) if np_dtype == np.uint16
         else rng.standard_normal((n, row_elems)).astype(np.float32))
    res = moe.moe_dispatch(None, to_dev(idx), e, g, sort=sort)
    xd = to_dev(x)
    rows_s = moe.moe_scatter_rows(xd, res.dst_pos, k)
    rows_g = moe.moe_gather_rows(xd, res.src_pair, k)
    _sync()
    ref = od.dispatch(idx, e, g, bool(sort))
    expect_g = od.gather_rows(x, ref["src_pair"], k)
    expect_s = od.scatter_rows(x, ref["dst_pos"], k)
    assert np.array_equal(expect_g, expect_s)
    assert np.array_equal(to_np(rows_s).view(np.uint8), expect_s.view(np.uint8))
    assert np.array_equal(to_np(rows_g).view(np.uint8), expect_g.view(np.uint8))


def test_scatter_rows_fp8_scales_as_bytes():
    cfg = CONFIGS["segment"].with_tokens(100)
    inp = make_inputs(cfg)
    idx = np.stack([np.random.default_rng(t).permutation(256)[:8] for t in range(100)]).astype(np.int32)
    res = moe.moe_dispatch(None, to_dev(idx), 256, 8, sort=0)
    rows = moe.moe_scatter_rows(to_dev(inp["x"]), res.dst_pos, 8)
    scales = moe.moe_scatter_rows(to_dev(inp["x_scales"]), res.dst_pos, 8)
    _sync()
    ref = od.dispatch(idx, 256, 8, False, x=inp["x"], x_scales=inp["x_scales"])
    assert np.array_equal(to_np(rows), ref["rows"])
    assert np.array_equal(to_np(scales), ref["row_scales"])
