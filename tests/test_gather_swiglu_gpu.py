"""SwiGLU experts over rows in any order (per-row expert ids) against the
oracle's row-by-row definition (oracle.swiglu.swiglu_rows); tolerance in
tests.gpu_util.check_swiglu."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from oracle import codecs
from oracle.combine import combine_f64
from oracle.swiglu import swiglu_combine, swiglu_rows
from tests.gpu_util import (DEV, check_swiglu, combine_check_all_tokens, per_expert_oracle, to_dev,
                            to_np)
from workloads import DECODE_FFN, make_inputs, make_swiglu_weights_device

pytestmark = pytest.mark.gpu


def _bf16(a):
    return codecs.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _weights(rng, e, d, f, std=0.05):
    return (_bf16(rng.standard_normal((e, f, d)) * std), _bf16(rng.standard_normal((e, f, d)) * std),
            _bf16(rng.standard_normal((e, d, f)) * std))


def _run(rows, experts, w, y=None):
    out = moe.moe_gather_swiglu(to_dev(rows), to_dev(np.asarray(experts, np.int32)),
                                *map(to_dev, w), y=y)
    torch.cuda.synchronize()
    return to_np(out)


@pytest.mark.parametrize("e,d,f,counts", [
    (4, 128, 128, [5, 0, 1, 31]),              # empty expert, 1 row, two passes (16 + 15)
    (8, 256, 384, [16, 17, 0, 3, 48, 1, 0, 9]),  # exact pass, pass + 1, three passes
    (3, 384, 256, [7, 33, 2]),                 # K = 384: three 128-chunks on gate/up
    (2, 640, 128, [20, 4]),                    # five chunks; down has one chunk (K = 128)
    (16, 128, 512, [1] * 16),                  # one row per expert, partial down group
    (1, 512, 256, [70]),                       # a single expert, five passes
    (2, 2432, 1152, [20, 3]),                  # K not a multiple of the 1024-wide row stage
])
def test_gather_swiglu_small(e, d, f, counts):
    rng = np.random.default_rng(d + 7 * f + e)
    experts = rng.permutation(np.repeat(np.arange(e), counts)).astype(np.int32)   # unsorted
    rows = _bf16(rng.standard_normal((experts.size, d)))
    w = _weights(rng, e, d, f)
    got = _run(rows, experts, w)
    ref = swiglu_rows(rows, experts, *w)
    check_swiglu(got, ref, experts, what=f"E={e} D={d} F={f}")


def test_gather_swiglu_matches_grouped_rows_either_order():
    """The same rows in expert-major order and shuffled: each row's output
    depends only on the row and its expert."""
    rng = np.random.default_rng(3)
    e, d, f = 6, 256, 256
    experts = np.repeat(np.arange(e), [3, 20, 0, 1, 40, 9]).astype(np.int32)
    rows = _bf16(rng.standard_normal((experts.size, d)))
    w = _weights(rng, e, d, f)
    perm = rng.permutation(experts.size)
    a = _run(rows, experts, w)
    b = _run(rows[perm], experts[perm], w)
    assert np.array_equal(a[perm], b)
    check_swiglu(a, swiglu_rows(rows, experts, *w), experts, what="grouped order")


def test_gather_swiglu_skips_out_of_range_ids():
    rng = np.random.default_rng(4)
    e, d, f = 3, 128, 128
    experts = np.array([0, -1, 2, 3, 1, 1, 99, 0, -7, 2], np.int32)
    rows = _bf16(rng.standard_normal((experts.size, d)))
    w = _weights(rng, e, d, f)
    y = torch.full((experts.size, d), 7.0, dtype=torch.bfloat16, device=DEV)
    got = _run(rows, experts, w, y=y)
    bad = (experts < 0) | (experts >= e)
    assert (codecs.bf16_bits_to_f32(got[bad]) == 7.0).all()
    ok = ~bad
    check_swiglu(got[ok], swiglu_rows(rows[ok], experts[ok], *w), experts[ok], what="in range")


def test_gather_swiglu_deterministic_and_empty():
    rng = np.random.default_rng(5)
    e, d, f = 4, 256, 128
    experts = rng.integers(0, e, 90).astype(np.int32)
    rows = _bf16(rng.standard_normal((90, d)))
    w = _weights(rng, e, d, f)
    assert np.array_equal(_run(rows, experts, w), _run(rows, experts, w))
    y = moe.moe_gather_swiglu(torch.empty((0, d), dtype=torch.bfloat16, device=DEV),
                              torch.empty(0, dtype=torch.int32, device=DEV), *map(to_dev, w))
    assert y.shape == (0, d)


def test_decode_layer_with_experts_full_size():
    """Decode with real experts: N=128, D=7168, E=256, top-8, unsorted identity
    layout, F=2048.  Route + unsorted dispatch -> per-row SwiGLU reading the
    rows where the dispatch left them -> combine.  Every row (all active
    experts) is checked against the oracle, each expert's weights copied back
    in turn; the combine is checked on every token on the GPU's own y."""
    cfg = DECODE_FFN
    inp = make_inputs(cfg)
    w = make_swiglu_weights_device(cfg)
    idx, tw, res = moe.moe_route_dispatch(to_dev(inp["logits"]), to_dev(inp["x"]), cfg.top_k,
                                          cfg.n_segments, cfg.renormalize, cfg.sort, cfg.sort_cutoff)
    assert not res.sorted
    y = moe.moe_gather_swiglu(res.rows, res.row_expert, w["w_gate"], w["w_up"], w["w_down"])
    out = moe.moe_combine(y, res.dst_pos, tw)
    torch.cuda.synchronize()
    rexp = to_np(res.row_expert)
    assert np.array_equal(rexp, to_np(idx).reshape(-1))     # identity layout: row t*k+j
    rows = to_np(res.rows)

    def fetch(e):
        return [w[nm][e:e + 1].view(torch.int16).cpu().numpy().view(np.uint16)
                for nm in ("w_gate", "w_up", "w_down")]

    ref = per_expert_oracle(lambda sel, local, ops: swiglu_rows(rows[sel], local, *ops), rexp, fetch)
    check_swiglu(to_np(y), ref, rexp, what="decode experts, every row")
    combine_check_all_tokens(out, y, res.dst_pos, tw, cfg.top_k, True, what="decode combine")


def test_gather_swiglu_multi_workgroup_grouping():
    """300 experts (> 256) and 5000 rows (> 4096): the grouping of the ids
    takes the multi-workgroup counting sort instead of the one-workgroup one."""
    rng = np.random.default_rng(6)
    e, d, f = 300, 128, 128
    experts = rng.integers(0, e, 5000).astype(np.int32)
    experts[:40] = 7                                   # one expert with three passes
    rows = _bf16(rng.standard_normal((experts.size, d)))
    w = _weights(rng, e, d, f)
    got = _run(rows, experts, w)
    check_swiglu(got, swiglu_rows(rows, experts, *w), experts, what="E=300 R=5000")


# ------------------------------------------------------------------ the combine fused in

def check_fused(got, ref, what=""):
    """got float32 [N, D] from the GPU, ref float64 from oracle.swiglu.swiglu_combine:
    the expert FFN tolerance (2e-2 of max(|o|, rms of the token's row)), the
    k weighted terms and the residual summed in fp32 on the GPU."""
    g = np.asarray(got, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    bad = np.abs(g - ref) > 2e-2 * np.maximum(np.abs(ref), rms)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} elements outside 2e-2"
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= 5e-3, f"{what}: relative error {rel:.3e}"


@pytest.mark.parametrize("n,k,e,d,f,shuffle", [
    (12, 4, 5, 256, 256, True),       # rows in a shuffled layout, row_pair given
    (40, 2, 3, 384, 128, False),      # identity layout (row_pair null), K = 384 path
    (7, 8, 16, 128, 512, True),
    (33, 1, 2, 512, 256, False),      # k = 1
])
def test_gather_swiglu_combine_small(n, k, e, d, f, shuffle):
    rng = np.random.default_rng(n * 31 + k)
    r = n * k
    experts = rng.integers(0, e, r).astype(np.int32)
    rows = _bf16(rng.standard_normal((r, d)))
    w = _weights(rng, e, d, f)
    tw = rng.uniform(0.05, 1.0, (n, k)).astype(np.float32)
    out0 = rng.standard_normal((n, d)).astype(np.float32)          # a residual to add into
    row_pair = rng.permutation(r).astype(np.int32) if shuffle else np.arange(r, dtype=np.int32)
    out = to_dev(out0.copy())
    moe.moe_gather_swiglu_combine(to_dev(rows), to_dev(experts), to_dev(tw), *map(to_dev, w),
                                  row_pair=to_dev(row_pair) if shuffle else None, out=out)
    torch.cuda.synchronize()
    ref = swiglu_combine(rows, experts, row_pair, tw, k, *w, out0=out0)
    check_fused(to_np(out), ref, what=f"N={n} k={k} E={e} D={d} F={f}")


def test_gather_swiglu_combine_skips_rows_without_pair_or_expert():
    rng = np.random.default_rng(8)
    n, k, e, d, f = 6, 2, 3, 128, 128
    experts = rng.integers(0, e, n * k).astype(np.int32)
    experts[3] = -1                                     # no expert
    row_pair = np.arange(n * k, dtype=np.int32)
    row_pair[5] = n * k + 7                             # no pair
    rows = _bf16(rng.standard_normal((n * k, d)))
    w = _weights(rng, e, d, f)
    tw = rng.uniform(0.1, 1.0, (n, k)).astype(np.float32)
    out = moe.moe_gather_swiglu_combine(to_dev(rows), to_dev(experts), to_dev(tw), *map(to_dev, w),
                                        row_pair=to_dev(row_pair))
    torch.cuda.synchronize()
    keep = np.ones(n * k, bool)
    keep[[3, 5]] = False
    ref = swiglu_combine(rows[keep], experts[keep], row_pair[keep], tw, k, *w)
    check_fused(to_np(out), ref, what="skipped rows")


def test_decode_layer_fused_combine_full_size():
    """The decode layer with the combine fused into the down product (N=128,
    D=7168, E=256, top-8, F=2048, unsorted identity layout).  Three tokens
    against the oracle (their 24 rows, the experts' weights copied back); all
    tokens against the unfused path (per-row FFN in bf16, then the combine in
    fp32), which differs only by the bf16 rounding of y: at most 2^-8 of
    sum_j |w_j y_j| per element, plus fp32 sums."""
    cfg = DECODE_FFN
    inp = make_inputs(cfg)
    w = make_swiglu_weights_device(cfg)
    idx, tw, res = moe.moe_route_dispatch(to_dev(inp["logits"]), to_dev(inp["x"]), cfg.top_k,
                                          cfg.n_segments, cfg.renormalize, cfg.sort, cfg.sort_cutoff)
    fused = moe.moe_gather_swiglu_combine(res.rows, res.row_expert, tw, w["w_gate"], w["w_up"],
                                          w["w_down"], row_pair=res.src_pair)
    y = moe.moe_gather_swiglu(res.rows, res.row_expert, w["w_gate"], w["w_up"], w["w_down"])
    unfused = moe.moe_combine(y, res.dst_pos, tw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    k = cfg.top_k
    yf = codecs.bf16_bits_to_f32(to_np(y)).astype(np.float64)
    mag = combine_f64(np.abs(yf), to_np(res.dst_pos), np.abs(to_np(tw)), k)
    diff = np.abs(to_np(fused).astype(np.float64) - to_np(unfused).astype(np.float64))
    assert (diff <= 2.0 ** -8 * mag + 1e-6 * mag + 1e-30).all(), float(np.max(diff - 2.0 ** -8 * mag))
    toks = np.array([0, 57, 127])
    rexp = to_np(res.row_expert)
    sel_rows = np.concatenate([np.arange(t * k, (t + 1) * k) for t in toks])   # identity layout
    chosen = np.unique(rexp[sel_rows])
    host = {nm: v.index_select(0, torch.from_numpy(chosen).to(DEV)).view(torch.int16).cpu()
            .numpy().view(np.uint16) for nm, v in w.items()}
    local = np.searchsorted(chosen, rexp[sel_rows])
    tw_np = to_np(tw)
    # the three tokens renumbered 0..2 with their own rows, pairs and weights
    row_pair = np.arange(toks.size * k)
    ref = swiglu_combine(to_np(res.rows)[sel_rows], local, row_pair, tw_np[toks], k,
                         host["w_gate"], host["w_up"], host["w_down"])
    check_fused(to_np(fused)[toks], ref, what="decode fused combine")


def test_gather_swiglu_max_experts():
    """E = 1024 (the library's maximum): one plan thread per expert, many empty
    experts, a few with several passes."""
    rng = np.random.default_rng(9)
    e, d, f = 1024, 128, 128
    experts = rng.integers(0, e, 2000).astype(np.int32)
    experts[:50] = 1023                                  # the last expert, four passes
    experts[50:70] = 0
    rows = _bf16(rng.standard_normal((experts.size, d)))
    w = _weights(rng, e, d, f)
    got = _run(rows, experts, w)
    check_swiglu(got, swiglu_rows(rows, experts, *w), experts, what="E=1024")


def test_gather_swiglu_random_shapes():
    """A seeded sweep of 12 shapes: D and F over multiples of 128 (both chunk
    widths), expert counts from 1 to 40, row counts from 1 to 700 with
    Zipf-like skew, some ids out of range."""
    master = np.random.default_rng(11)
    for case in range(12):
        e = int(master.integers(1, 41))
        d = 128 * int(master.integers(1, 7))
        f = 128 * int(master.integers(1, 5))
        r = int(master.integers(1, 701))
        p = 1.0 / np.arange(1, e + 1) ** 1.1
        experts = master.choice(e, r, p=p / p.sum()).astype(np.int32)
        experts[master.random(r) < 0.03] = -1
        rows = _bf16(master.standard_normal((r, d)))
        w = _weights(master, e, d, f)
        y0 = torch.full((r, d), 3.0, dtype=torch.bfloat16, device=DEV)
        got = _run(rows, experts, w, y=y0)
        ok = experts >= 0
        assert (codecs.bf16_bits_to_f32(got[~ok]) == 3.0).all(), case
        if ok.any():
            check_swiglu(got[ok], swiglu_rows(rows[ok], experts[ok], *w), experts[ok],
                         what=f"case {case}: E={e} D={d} F={f} R={r}")
