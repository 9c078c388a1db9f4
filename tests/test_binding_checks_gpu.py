"""The Python binding rejects undersized or mis-shaped tensors with ValueError
before any launch (the C ABI takes raw pointers and cannot see tensor sizes).
Each case pre-fills the buffers the call would write and checks, after the
error, that nothing was written."""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _i32(*shape, fill=-7):
    return torch.full(shape, fill, dtype=torch.int32, device=DEV)


def _untouched(*ts, fill=-7):
    torch.cuda.synchronize()
    for t in ts:
        assert bool((t == fill).all()), "a rejected call wrote into an output"


def _idx(n=16, e=8, k=2):
    rng = np.random.default_rng(0)
    return torch.from_numpy(np.stack([rng.permutation(e)[:k] for _ in range(n)]).astype(np.int32)).to(DEV)


def test_dispatch_rejects_short_outputs_and_scales():
    idx = _idx()
    x = torch.zeros((16, 128), dtype=torch.bfloat16, device=DEV)
    good = moe.moe_dispatch(x, idx, 8, 2, sort=1)
    torch.cuda.synchronize()
    for name, short in (("dst_pos", _i32(31)), ("src_pair", _i32(31)), ("expert_offsets", _i32(8)),
                        ("expert_counts", _i32(7)), ("segment_offsets", _i32(2)),
                        ("row_expert", _i32(16))):
        bad = moe.DispatchResult(**{**good.__dict__, name: short})
        with pytest.raises(ValueError, match=name):
            moe.moe_dispatch(x, idx, 8, 2, sort=1, out=bad)
        _untouched(short)
    rows = torch.full((31, 128), 7, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="rows"):
        moe.moe_dispatch(x, idx, 8, 2, sort=1, out=moe.DispatchResult(**{**good.__dict__, "rows": rows}))
    _untouched(rows, fill=7)
    # fp8 payload with a scale tensor of the wrong width
    x8 = torch.zeros((16, 256), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="x_scales"):
        moe.moe_dispatch(x8, idx, 8, 2, sort=1, x_scales=torch.ones((16, 1), device=DEV))
    with pytest.raises(ValueError, match="x"):
        moe.moe_dispatch(x[:15], idx, 8, 2, sort=1)


def test_route_dispatch_rejects_short_outputs():
    logits = torch.randn((16, 8), device=DEV)
    x = torch.zeros((16, 64), dtype=torch.bfloat16, device=DEV)
    _, _, good = moe.moe_route_dispatch(logits, x, 2, 1, sort=1)
    torch.cuda.synchronize()
    short = _i32(30)
    with pytest.raises(ValueError, match="dst_pos"):
        moe.moe_route_dispatch(logits, x, 2, 1, sort=1,
                               out=moe.DispatchResult(**{**good.__dict__, "dst_pos": short}))
    _untouched(short)
    tw = torch.full((16, 3), -7.0, device=DEV)
    with pytest.raises(ValueError, match="topk_w"):
        moe.moe_route_dispatch(logits, x, 2, 1, sort=1, topk_w=tw)
    _untouched(tw, fill=-7.0)


def test_combine_rejects_wrong_out_shape():
    y = torch.ones((32, 64), dtype=torch.bfloat16, device=DEV)
    dst = torch.arange(32, dtype=torch.int32, device=DEV)
    w = torch.full((16, 2), 0.5, device=DEV)
    out = torch.full((16, 32), -7, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="out"):
        moe.moe_combine(y, dst, w, out=out)
    _untouched(out, fill=-7)
    with pytest.raises(ValueError):
        moe.moe_combine(y[:31], dst[:31], w)


def test_row_copies_reject_narrow_rows():
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    dst = torch.arange(16, dtype=torch.int32, device=DEV)
    rows = torch.full((16, 32), -7, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="row shape"):
        moe.moe_scatter_rows(x, dst, 2, rows=rows)
    with pytest.raises(ValueError, match="rows"):
        moe.moe_gather_rows(x, dst, 2, rows=rows)
    _untouched(rows, fill=-7)


def test_dequant_rejects_wrong_scales_and_out():
    rows = torch.zeros((4, 256), dtype=torch.uint8, device=DEV)
    out = torch.full((4, 128), -7, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="row_scales"):
        moe.moe_dequant_rows(rows, torch.ones((4, 1), device=DEV))
    with pytest.raises(ValueError, match="out"):
        moe.moe_dequant_rows(rows, torch.ones((4, 2), device=DEV), out=out)
    _untouched(out, fill=-7)


def test_grouped_swiglu_rejects_inconsistent_weights_and_offsets():
    e, d, f = 2, 64, 128
    rows = torch.zeros((10, d), dtype=torch.bfloat16, device=DEV)
    wg = torch.zeros((e, f, d), dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros((e, d, f), dtype=torch.bfloat16, device=DEV)
    offs = torch.tensor([0, 4, 10], dtype=torch.int32, device=DEV)
    y = torch.full((10, d), -7, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="inconsistent"):
        moe.moe_grouped_swiglu(rows, offs, wg, wg[:, :64].contiguous(), wd, y=y)   # short w_up
    with pytest.raises(ValueError, match="inconsistent"):
        moe.moe_grouped_swiglu(rows, offs, wg, wg, wd[:, :, :64].contiguous(), y=y)  # short w_down
    with pytest.raises(ValueError, match="inconsistent"):
        moe.moe_grouped_swiglu(rows, offs[:2], wg, wg, wd, y=y)              # E offsets, not E+1
    with pytest.raises(ValueError, match="inconsistent"):
        moe.moe_grouped_swiglu(rows[:, :32].contiguous(), offs, wg, wg, wd)  # D of rows != D of weights
    _untouched(y, fill=-7)
