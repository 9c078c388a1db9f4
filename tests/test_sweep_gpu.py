"""Seeded random sweep of shapes through route -> dispatch -> combine, and the
large-problem paths (chunk growth above 1M pairs), against the oracle."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from oracle import codecs, dispatch as od
from oracle.route import route_topk as oracle_route
from tests.gpu_util import as_f32, check_combine, check_weights, combine_reference, to_dev, to_np

pytestmark = pytest.mark.gpu


def _divisors(e):
    return [g for g in range(1, e + 1) if e % g == 0]


def _case(seed):
    rng = np.random.default_rng(seed)
    e = int(rng.choice([1, 2, 3, 8, 16, 60, 64, 100, 128, 256, 512, 1000, 1024]))
    k = int(rng.integers(1, min(e, 64) + 1))
    n = int(rng.choice([0, 1, 2, 7, 63, 64, 65, 333, 1000, 2500, 5000]))
    g = int(rng.choice(_divisors(e)))
    d = int(rng.choice([1, 3, 8, 24, 40, 128, 136, 300]))
    dtype = str(rng.choice(["f32", "bf16"]))
    sort = int(rng.choice([-1, 0, 1]))
    cutoff = int(rng.choice([0, 1, 64, 256]))
    return rng, e, k, n, g, d, dtype, sort, cutoff


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes(seed):
    rng, e, k, n, g, d, dtype, sort, cutoff = _case(seed)
    logits = rng.standard_normal((n, e)).astype(np.float32)
    xf = rng.standard_normal((n, d)).astype(np.float32)
    x = codecs.f32_to_bf16_bits(xf) if dtype == "bf16" else xf
    if n == 0:
        idx = torch.empty((0, k), dtype=torch.int32, device="cuda:0")
        w = torch.empty((0, k), dtype=torch.float32, device="cuda:0")
    else:
        idx, w = moe.moe_route_topk(to_dev(logits), k)
    res = moe.moe_dispatch(to_dev(x) if n else torch.empty((0, d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device="cuda:0"),
                           idx, e, g, sort=sort, sort_cutoff=cutoff)
    torch.cuda.synchronize()
    if n == 0:
        assert (to_np(res.expert_offsets) == 0).all()
        return
    oi, ow = oracle_route(logits, k)
    assert np.array_equal(to_np(idx), oi)
    check_weights(to_np(w), ow)
    assert res.sorted == od.resolve_sorted(sort, n, cutoff)
    ref = od.dispatch(oi, e, g, res.sorted, x=x)
    for name in ("expert_counts", "expert_offsets", "segment_offsets", "src_pair", "dst_pos", "row_expert"):
        assert np.array_equal(to_np(getattr(res, name)), ref[name]), name
    assert np.array_equal(to_np(res.rows).view(np.uint8), ref["rows"].view(np.uint8))
    out = moe.moe_combine(res.rows, res.dst_pos, w)
    torch.cuda.synchronize()
    exact, mag = combine_reference(as_f32(ref["rows"]), ref["dst_pos"], to_np(w), k)
    check_combine(to_np(out), exact, mag, dtype == "bf16", what=f"seed {seed}")


@pytest.mark.parametrize("sort,g", [(1, 1), (0, 4), (0, 1)])
def test_dispatch_beyond_a_million_pairs(sort, g):
    """NK = 1.6M pairs: the chunk size grows past 1024 pairs."""
    rng = np.random.default_rng(11)
    n, e, k = 200_000, 64, 8
    idx = np.argsort(rng.random((n, e)), axis=1)[:, :k].astype(np.int32)
    x = rng.integers(0, 2**16, (n, 8), dtype=np.uint16)
    res = moe.moe_dispatch(to_dev(x), to_dev(idx), e, g, sort=sort)
    torch.cuda.synchronize()
    ref = od.dispatch(idx, e, g, bool(sort))
    for name in ("expert_counts", "expert_offsets", "segment_offsets", "src_pair", "dst_pos", "row_expert"):
        assert np.array_equal(to_np(getattr(res, name)), ref[name]), name
    rows = to_np(res.rows)
    sample = rng.integers(0, n * k, 5000)
    assert np.array_equal(rows[sample], x[ref["src_pair"][sample] // k])


@pytest.mark.parametrize("renorm", [True, False])
def test_route_many_tokens(renorm):
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((50_000, 256)).astype(np.float32)
    idx, w = moe.moe_route_topk(to_dev(logits), 8, renorm)
    torch.cuda.synchronize()
    oi, ow = oracle_route(logits, 8, renorm)
    assert np.array_equal(to_np(idx), oi)
    check_weights(to_np(w), ow)
