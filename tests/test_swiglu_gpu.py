"""Grouped SwiGLU expert FFN (matrix cores) against the oracle; tolerance in
tests.gpu_util.check_swiglu."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from oracle import codecs, dispatch as od
from oracle.swiglu import swiglu_hidden, swiglu_rows
from tests.gpu_util import DEV, check_swiglu, combine_check_all_tokens, tile_rows, to_dev, to_np
from workloads import CONFIGS, make_inputs, make_swiglu_weights_device

pytestmark = pytest.mark.gpu


def _bf16(a):
    return codecs.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("e,d,f,offs", [
    (4, 128, 192, [0, 0, 130, 131, 300]),     # empty expert, 1-row expert, ragged tiles
    (4, 64, 128, [0, 0, 0, 0, 2]),            # the gather_mm_e4_i64_o128 shape: 2 rows on expert 3
    (3, 192, 64, [0, 129, 129, 257]),
    (8, 256, 320, [0, 40, 80, 300, 301, 302, 560, 700, 1000]),
])
def test_grouped_swiglu_small(e, d, f, offs):
    rng = np.random.default_rng(d + f)
    n_rows = offs[-1]
    rows = _bf16(rng.standard_normal((n_rows, d)))
    wg = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wu = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.05)
    y = moe.moe_grouped_swiglu(to_dev(rows), to_dev(np.array(offs, np.int32)), to_dev(wg), to_dev(wu), to_dev(wd))
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(e), np.diff(offs))
    ref = swiglu_rows(rows, experts, wg, wu, wd)
    check_swiglu(to_np(y), ref, experts, what=f"E={e} D={d} F={f}")


def test_grouped_swiglu_does_not_touch_rows_outside_offsets():
    rng = np.random.default_rng(1)
    e, d, f = 2, 64, 64
    rows = _bf16(rng.standard_normal((40, d)))
    w = [_bf16(rng.standard_normal(s) * 0.05) for s in ((e, f, d), (e, f, d), (e, d, f))]
    y = torch.full((40, d), 7.0, dtype=torch.bfloat16, device=DEV)
    moe.moe_grouped_swiglu(to_dev(rows), to_dev(np.array([0, 10, 30], np.int32)), *map(to_dev, w), y=y)
    torch.cuda.synchronize()
    yy = codecs.bf16_bits_to_f32(to_np(y))
    assert (yy[30:] == 7.0).all()


def split_tile_rows(offs, n_rows: int, n_col_tiles: int, k_stages: int, n_cus: int):
    """Host mirror of the grouped kernel's tile plan, for the test only: the
    row ranges of the tiles of a launch's last, partial round, which the
    kernel splits along K.  Row tiles are 256 rows from each expert's first
    row; tiles run in groups of 8 row tiles x all column tiles, row tiles
    fastest; whole rounds hold n_cus tiles.  Returns [(row0, row_end)] and the
    number of K parts (1: no split)."""
    tiles_rows = []
    offs = np.asarray(offs, np.int64)
    for e in range(offs.size - 1):
        for r0 in range(int(offs[e]), int(offs[e + 1]), 256):
            tiles_rows.append((r0, int(offs[e + 1])))
    m_real = len(tiles_rows)
    tiles = m_real * n_col_tiles
    full = tiles // n_cus * n_cus
    tail = tiles - full
    split = 1
    if tail > 0 and k_stages % 2 == 0:
        split = max(1, min(n_cus // tail, 8, k_stages // 2))
    out = set()
    for t in range(full, tiles):
        g = t // (8 * n_col_tiles)
        m0 = g * 8
        gm = min(8, m_real - m0)
        i = t - g * 8 * n_col_tiles
        out.add(tiles_rows[m0 + i % gm])
    return sorted(out), split


def test_mixtral_layer_full_size():
    """Route -> sorted dispatch -> grouped SwiGLU reading the rows in place ->
    combine, at N=8192, D=4096, E=8, k=2, F=14336.  Checked against the
    oracle: one row of every 256-row tile of every expert plus each expert's
    last row (so every tile of both launches, including the K-split tiles of a
    last partial round), both in h (the gate/up launch's output, read from the
    workspace) and in y; the combine on every token."""
    cfg = CONFIGS["mixtral"]
    inp = make_inputs(cfg)
    w = make_swiglu_weights_device(cfg)
    idx, tw = moe.moe_route_topk(to_dev(inp["logits"]), cfg.top_k)
    res = moe.moe_dispatch(to_dev(inp["x"]), idx, cfg.n_experts, 1, sort=-1, sort_cutoff=cfg.sort_cutoff)
    assert res.sorted                                    # N = 8192 > cutoff 256
    n_rows, f, d = cfg.n_tokens * cfg.top_k, cfg.ffn, cfg.hidden
    ws = torch.empty(moe.moe_grouped_swiglu_workspace_bytes(n_rows, cfg.n_experts, d, f),
                     dtype=torch.uint8, device=DEV)
    y = moe.moe_grouped_swiglu(res.rows, res.expert_offsets, w["w_gate"], w["w_up"], w["w_down"],
                               workspace=ws)
    out = moe.moe_combine(y, res.dst_pos, tw)
    torch.cuda.synchronize()
    h = ws[: n_rows * f * 2].view(torch.bfloat16).view(n_rows, f)     # h [R, F] opens the workspace
    offs = to_np(res.expert_offsets)
    sample = tile_rows(offs, 256, np.random.default_rng(0))
    n_cus = min(256, torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8)
    split_any = False
    for n_col_tiles, k_stages in ((f // 128, d // 64), (d // 256, f // 64)):
        ranges, split = split_tile_rows(offs, n_rows, n_col_tiles, k_stages, n_cus)
        split_any |= split > 1 and bool(ranges)
        for r0, r1 in ranges:                           # every last-round tile has a checked row
            assert np.any((sample >= r0) & (sample < min(r0 + 256, r1))), (r0, r1)
    assert split_any, "the full-size layer should exercise the K-split last round"
    rows = to_np(res.rows)[sample]
    experts = to_np(res.row_expert)[sample]
    host_w = {k: v.view(torch.int16).cpu().numpy().view(np.uint16) for k, v in w.items()}
    ref_h = swiglu_hidden(rows, experts, host_w["w_gate"], host_w["w_up"])
    check_swiglu(to_np(h)[sample], ref_h, experts, what="mixtral h")
    ref = swiglu_rows(rows, experts, host_w["w_gate"], host_w["w_up"], host_w["w_down"])
    check_swiglu(to_np(y)[sample], ref, experts, what="mixtral y")
    # the combine over the GEMM output, every token, on the GPU's own y
    combine_check_all_tokens(out, y, res.dst_pos, tw, cfg.top_k, True, what="mixtral combine")


def test_grouped_swiglu_many_experts():
    """E = 300: the device's tile count scans the offsets 64 experts at a time; many
    experts are empty and a few span several 256-row tiles."""
    rng = np.random.default_rng(300)
    e, d, f = 300, 128, 192
    sizes = rng.choice([0, 0, 0, 1, 3, 17, 255, 256, 257, 600], size=e)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    n_rows = int(offs[-1])
    rows = _bf16(rng.standard_normal((n_rows, d)))
    wg = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wu = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.05)
    y = moe.moe_grouped_swiglu(to_dev(rows), to_dev(offs), to_dev(wg), to_dev(wu), to_dev(wd))
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(e), sizes)
    ref = swiglu_rows(rows, experts, wg, wu, wd)
    check_swiglu(to_np(y), ref, experts, what="E=300")


@pytest.mark.parametrize("offs", [[0, 100, 50, 200, 180, 260], [20, 100, 50, 200, 180, 260],
                                  [-5, 70, 400, 30, 500, 10]])
def test_grouped_swiglu_offsets_outside_the_contract(offs):
    """Offsets that start above 0, decrease or run past the rows are clamped into
    [0, R] and made non-decreasing (lo_0 = clamp(offs[0]), hi_e = clamp(offs[e+1],
    lo_e, R)): rows inside those ranges get their expert's FFN, the rest of y is
    untouched."""
    rng = np.random.default_rng(len(offs) + offs[0] + 7)
    e, d, f, n_rows = len(offs) - 1, 64, 128, 300
    rows = _bf16(rng.standard_normal((n_rows, d)))
    wg = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wu = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.05)
    y = torch.full((n_rows, d), 7.0, dtype=torch.bfloat16, device=DEV)
    moe.moe_grouped_swiglu(to_dev(rows), to_dev(np.array(offs, np.int32)), to_dev(wg), to_dev(wu),
                           to_dev(wd), y=y)
    torch.cuda.synchronize()
    experts = np.full(n_rows, -1)
    lo = min(max(offs[0], 0), n_rows)
    for j in range(e):
        hi = min(max(offs[j + 1], lo), n_rows)
        experts[lo:hi] = j
        lo = hi
    yy = codecs.bf16_bits_to_f32(to_np(y))
    inside = experts >= 0
    assert (yy[~inside] == 7.0).all()
    ref = swiglu_rows(rows[inside], experts[inside], wg, wu, wd)
    check_swiglu(to_np(y)[inside], ref, experts[inside], what=f"offsets {offs}")


def test_grouped_swiglu_split_tiles_deterministic():
    """Few tiles over a long K: every tile of both launches is split into K parts
    (up to 8) whose fp32 partials are summed in part order by the last part to
    finish.  Parity with the oracle, and bit-identical output on a second call."""
    rng = np.random.default_rng(8)
    e, d, f = 3, 1024, 512
    offs = np.array([0, 130, 130, 300], np.int32)
    n_rows = int(offs[-1])
    rows = _bf16(rng.standard_normal((n_rows, d)))
    wg = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wu = _bf16(rng.standard_normal((e, f, d)) * 0.05)
    wd = _bf16(rng.standard_normal((e, d, f)) * 0.05)
    args = (to_dev(rows), to_dev(offs), to_dev(wg), to_dev(wu), to_dev(wd))
    y1 = moe.moe_grouped_swiglu(*args)
    y2 = moe.moe_grouped_swiglu(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    experts = np.repeat(np.arange(e), np.diff(offs))
    ref = swiglu_rows(rows, experts, wg, wu, wd)
    check_swiglu(to_np(y1), ref, experts, what="split tiles")
