"""fp8 block-scaled grouped expert GEMM (matrix cores) against the oracle.

Tolerance.  The oracle's value is exact up to float64 rounding.  The kernel
multiplies fp8 codes on the matrix cores (v_mfma_f32_32x32x16_fp8_fp8), whose
16-term dot products are not accumulated as exactly as fp32 would: on MI355X a
single instruction was measured off by up to about 2^-14 of its largest
outputs.  The per-block partial sums are then scaled and accumulated in fp32
over K/128 blocks and rounded once to bfloat16.  Per element:

    |got - exact| <= 2^-8 * |exact| + 2^-11 * magnitude

where magnitude is the sum of the absolute values of every term
(oracle.gemm_fp8.gemm_fp8_magnitude).  2^-8 covers the bf16 rounding (half an
ulp is at most 2^-9 of the value), 2^-11 the accumulation, 8x above the
measured instruction error.  A dropped block, a wrong scale or a wrong
expert's weights moves an output by a sizeable fraction of its magnitude and
fails.
"""
import numpy as np
import pytest
import torch

import combine_moe_route_topk_amd as moe
from oracle import codecs
from oracle.gemm_fp8 import gemm_fp8_magnitude, gemm_fp8_rows
from tests.gpu_util import DEV, per_expert_oracle, tile_rows, to_dev, to_np
from workloads import CONFIGS, FP8_GEMM_N, make_fp8_expert_weights_device, make_inputs

pytestmark = pytest.mark.gpu


def _codes(rng, shape):
    q = rng.integers(0, 256, shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x30                 # no NaN codes
    return q


def check_fp8_gemm(got_bits, rows, sx, experts, w, sw, what):
    got = codecs.bf16_bits_to_f32(got_bits).astype(np.float64)
    exact = gemm_fp8_rows(rows, sx, experts, w, sw)
    mag = gemm_fp8_magnitude(rows, sx, experts, w, sw)
    err = np.abs(got - exact)
    bound = 2.0 ** -8 * np.abs(exact) + 2.0 ** -11 * mag
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside the bound; worst "
                           f"err/magnitude {float(np.max(err / np.maximum(mag, 1e-300))):.3g}")
    return float(np.max((err - 2.0 ** -8 * np.abs(exact)).clip(0) / np.maximum(mag, 1e-300)))


@pytest.mark.parametrize("e,k,n,offs", [
    (4, 256, 256, [0, 0, 70, 71, 200]),       # empty expert, 1-row expert, 2 row tiles, ragged
    (3, 384, 128, [0, 64, 64, 130]),          # odd number of K blocks, exact 64-row tile
    (2, 128, 384, [0, 5, 9]),                 # a single K block, 3 column tiles
    (8, 512, 256, [0, 40, 41, 100, 100, 170, 250, 251, 300]),
])
def test_grouped_gemm_fp8_small(e, k, n, offs):
    rng = np.random.default_rng(k + n + e)
    r = offs[-1]
    rows = _codes(rng, (r, k))
    sx = rng.uniform(1e-3, 1e-1, (r, k // 128)).astype(np.float32)
    w = _codes(rng, (e, n, k))
    sw = rng.uniform(1e-3, 1e-1, (e, n // 128, k // 128)).astype(np.float32)
    y = moe.moe_grouped_gemm_fp8(to_dev(rows), to_dev(sx), to_dev(np.array(offs, np.int32)),
                                 to_dev(w), to_dev(sw))
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(e), np.diff(offs))
    check_fp8_gemm(to_np(y), rows, sx, experts, w, sw, f"E={e} K={k} N={n}")


def test_grouped_gemm_fp8_leaves_rows_outside_offsets():
    rng = np.random.default_rng(5)
    e, k, n = 2, 128, 128
    rows = _codes(rng, (30, k))
    sx = np.ones((30, 1), np.float32)
    w = _codes(rng, (e, n, k))
    sw = np.full((e, 1, 1), 0.01, np.float32)
    y = torch.full((30, n), 7.0, dtype=torch.bfloat16, device=DEV)
    moe.moe_grouped_gemm_fp8(to_dev(rows), to_dev(sx), to_dev(np.array([2, 10, 20], np.int32)),
                             to_dev(w), to_dev(sw), y=y)
    torch.cuda.synchronize()
    yy = codecs.bf16_bits_to_f32(to_np(y))
    assert (yy[:2] == 7.0).all() and (yy[20:] == 7.0).all()
    check_fp8_gemm(to_np(y)[2:20], rows[2:20], sx[2:20], np.repeat([0, 1], [8, 10]), w, sw, "inside")


def test_grouped_gemm_fp8_deterministic():
    rng = np.random.default_rng(6)
    e, k, n = 4, 512, 256
    offs = np.array([0, 50, 120, 121, 250], np.int32)
    args = [to_dev(_codes(rng, (250, k))), to_dev(rng.uniform(0.01, 1, (250, k // 128)).astype(np.float32)),
            to_dev(offs), to_dev(_codes(rng, (e, n, k))),
            to_dev(rng.uniform(0.01, 1, (e, n // 128, k // 128)).astype(np.float32))]
    a = moe.moe_grouped_gemm_fp8(*args)
    b = moe.moe_grouped_gemm_fp8(*args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_segment_workload_fp8_projection_full_size():
    """Segment-major workload (N=1024 tokens, D=7168 fp8 + 1x128 scales, E=256,
    top-8): routing, the sorted fp8 dispatch, then the fp8 grouped projection
    (N_out = 4096) reading the dispatched rows and scales in place.  Checked
    against the oracle on every output tile: one row of every 64-row tile of
    every expert plus each expert's last row, at four columns of every
    128-column tile (its first and last and two random ones)."""
    cfg = CONFIGS["segment"]
    inp = make_inputs(cfg)
    x = to_dev(inp["x"])
    xs = to_dev(inp["x_scales"])
    idx, tw, res = moe.moe_route_dispatch(to_dev(inp["logits"]), x, cfg.top_k, cfg.n_segments,
                                          cfg.renormalize, 1, cfg.sort_cutoff, x_scales=xs)
    assert res.sorted
    wt = make_fp8_expert_weights_device(cfg)
    y = moe.moe_grouped_gemm_fp8(res.rows, res.row_scales, res.expert_offsets, wt["w"],
                                 wt["w_scales"])
    torch.cuda.synchronize()
    assert tuple(y.shape) == (cfg.n_tokens * cfg.top_k, FP8_GEMM_N)
    offs = to_np(res.expert_offsets)
    rng = np.random.default_rng(0)
    sample = tile_rows(offs, 64, rng)
    experts = to_np(res.row_expert)[sample]
    cols = np.concatenate([np.unique(np.concatenate([[c, c + 127], c + rng.integers(1, 127, 2)]))
                           for c in range(0, FP8_GEMM_N, 128)])
    rows_s, sx_s, got = to_np(res.rows)[sample], to_np(res.row_scales)[sample], to_np(y)[sample][:, cols]

    def fetch(e):
        return wt["w"][e:e + 1].cpu().numpy(), wt["w_scales"][e:e + 1].cpu().numpy()

    def oracle(sel, local, ops):
        w_e, sw_e = ops
        return np.stack([gemm_fp8_rows(rows_s[sel], sx_s[sel], local, w_e, sw_e, cols=cols),
                         gemm_fp8_magnitude(rows_s[sel], sx_s[sel], local, w_e, sw_e, cols=cols)])

    both = per_expert_oracle(lambda sel, local, ops: oracle(sel, local, ops).transpose(1, 0, 2),
                             experts, fetch)
    exact, mag = both[:, 0], both[:, 1]
    g = codecs.bf16_bits_to_f32(got).astype(np.float64)
    err = np.abs(g - exact)
    bad = err > 2.0 ** -8 * np.abs(exact) + 2.0 ** -11 * mag
    assert not bad.any(), f"segment fp8 projection: {bad.sum()} of {bad.size} outside the bound"
    assert len(np.unique(experts)) == int(np.sum(np.diff(offs) > 0))     # every busy expert
