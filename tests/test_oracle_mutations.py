"""Each oracle pin catches a plausible mistake: a mutant of an oracle function
is swapped into the pin tests (CPU only), and the pins must fail for it."""
import numpy as np
import pytest

from oracle import codecs, combine as oc, dispatch as od, route as orr, swiglu as osw
from tests import (test_oracle_codecs as tc, test_oracle_combine as tcb,
                   test_oracle_dispatch as td, test_oracle_route as tr,
                   test_oracle_swiglu as tsw)
from tests.conftest import read_golden


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


# ------------------------------------------------------------------ routing mutants

def route_ties_high_index(logits, k, renormalize=True):
    """Mutant: among equal logits the higher expert index wins."""
    l = np.asarray(logits, np.float64) + 0.0
    e = l.shape[1]
    order = (e - 1) - np.argsort(-l[:, ::-1], axis=1, kind="stable")
    idx, w = orr.route_topk(logits, k, renormalize)
    sel = np.take_along_axis(l, order[:, :k], 1)
    ex = np.exp(sel - sel[:, :1])
    return order[:, :k].astype(np.int32), (ex / ex.sum(1, keepdims=True)).astype(np.float32)


def route_no_renormalise(logits, k, renormalize=True):
    """Mutant: always the full softmax."""
    return orr.route_topk(logits, k, False)


def route_signed_zero_ordered(logits, k, renormalize=True):
    """Mutant: -0.0 sorts below +0.0."""
    l = np.asarray(logits, np.float32).astype(np.float64)
    key = l - np.signbit(l) * (l == 0) * 1e-300
    order = np.argsort(-key, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l, order[:, :k], 1)
    ex = np.exp(sel - sel[:, :1])
    return idx, (ex / ex.sum(1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("mutant", [route_ties_high_index, route_no_renormalise, route_signed_zero_ordered])
def test_route_pins_catch(monkeypatch, mutant):
    monkeypatch.setattr(tr, "route_topk", mutant)
    results = []
    for t in (lambda: tr.test_golden_small(read_golden), tr.test_all_equal_logits,
              tr.test_descending_ramp_and_signed_zero, tr.test_k2_logistic_closed_form):
        try:
            t()
            results.append(False)
        except AssertionError:
            results.append(True)
    assert any(results), "no routing pin caught the mutant"


# ------------------------------------------------------------------ dispatch mutants

def perm_unstable(idx, n_experts, n_segments, sorted_):
    """Mutant: ties inside a bucket in reverse pair order."""
    flat = np.asarray(idx, np.int64).ravel()
    key = od.bucket_keys(idx, n_experts, n_segments, sorted_)
    q = np.arange(flat.size)
    src = np.lexsort((-q, key))
    dst = np.empty_like(src)
    dst[src] = q
    return src.astype(np.int32), dst.astype(np.int32), flat[src].astype(np.int32)


def perm_segment_modulo(idx, n_experts, n_segments, sorted_):
    """Mutant: segment of expert e taken as e % G instead of e // (E/G)."""
    flat = np.asarray(idx, np.int64).ravel()
    key = flat if sorted_ else flat % n_segments
    src = np.argsort(key, kind="stable")
    dst = np.empty_like(src)
    dst[src] = np.arange(src.size)
    return src.astype(np.int32), dst.astype(np.int32), flat[src].astype(np.int32)


@pytest.mark.parametrize("mutant", [perm_unstable, perm_segment_modulo])
def test_dispatch_pins_catch(monkeypatch, mutant):
    monkeypatch.setattr(od, "permutation", mutant)
    _fails(td.test_golden_small, read_golden)


def test_offsets_pin_catches_inclusive_scan(monkeypatch):
    monkeypatch.setattr(od, "expert_offsets", lambda c: np.concatenate([np.cumsum(c), [0]]).astype(np.int32))
    _fails(td.test_golden_small, read_golden)


def test_resolve_pin_catches_off_by_one(monkeypatch):
    def mutant(sort, n, cutoff):
        if sort in (0, 1):
            return bool(sort)
        return True if cutoff <= 0 else n >= cutoff
    monkeypatch.setattr(td.od, "resolve_sorted", mutant)
    _fails(td.test_resolve_sorted)


# ------------------------------------------------------------------ combine mutants

def combine_drop_last(y, dst_pos, w, k, tokens=None):
    """Mutant: the last slot is left out."""
    y = np.asarray(y)
    dst = np.asarray(dst_pos, np.int64).reshape(-1, k)
    ww = np.asarray(w, np.float32).astype(np.float64).reshape(-1, k)
    ts = np.arange(dst.shape[0]) if tokens is None else np.asarray(tokens)
    out = np.zeros((ts.size, y.shape[1]))
    for j in range(k - 1):
        out += ww[ts, j:j + 1] * y[dst[ts, j]]
    return out


def combine_weight_by_row(y, dst_pos, w, k, tokens=None):
    """Mutant: the weight is looked up by destination row instead of by pair."""
    y = np.asarray(y)
    dst = np.asarray(dst_pos, np.int64)
    wf = np.asarray(w, np.float32).astype(np.float64).ravel()
    n = dst.size // k
    ts = np.arange(n) if tokens is None else np.asarray(tokens)
    out = np.zeros((ts.size, y.shape[1]))
    for j in range(k):
        rows = dst.reshape(-1, k)[ts, j]
        out += wf[rows][:, None] * y[rows]
    return out


@pytest.mark.parametrize("mutant", [combine_drop_last, combine_weight_by_row])
def test_combine_pins_catch(monkeypatch, mutant):
    monkeypatch.setattr(tcb, "combine_f64", mutant)
    _fails(tcb.test_golden_small, read_golden)
    _fails(tcb.test_identity_experts_reproduce_input)


# ------------------------------------------------------------------ codec / expert mutants

def test_bf16_pin_catches_truncation(monkeypatch):
    def trunc(x):
        f = np.ascontiguousarray(np.asarray(x, np.float32))
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    monkeypatch.setattr(tc.codecs, "f32_to_bf16_bits", trunc)
    _fails(tc.test_f32_to_bf16_rne_vs_torch)


def test_fp8_pin_catches_wrong_bias(monkeypatch):
    table = codecs.fp8_e4m3fn_table() * 0.5          # as if the exponent bias were 8
    monkeypatch.setattr(tc.codecs, "fp8_bits_to_f64", lambda b: table[np.asarray(b, np.uint8)])
    _fails(tc.test_fp8_table_all_patterns_vs_torch)


def test_swiglu_pins_catch_sigmoid_for_silu(monkeypatch):
    monkeypatch.setattr(osw, "silu", lambda a: 1.0 / (1.0 + np.exp(-np.asarray(a, np.float64))))
    monkeypatch.setattr(tsw, "silu", osw.silu)
    _fails(tsw.test_silu_closed_forms)
    _fails(tsw.test_rows_match_pure_python_brute_force)


def _fused_mutant(kind):
    """Mutants of the fused combine: the weight of the transposed slot, the
    token taken as q % N instead of q // k, or y rounded to bf16 first."""
    def f(rows, experts, row_pair, topk_w, k, wg, wu, wd, out0=None):
        w = np.asarray(topk_w, np.float32).astype(np.float64).reshape(-1)
        n_tok = w.size // k
        y = osw.swiglu_rows_f64(rows, experts, wg, wu, wd)
        if kind == "round_y":
            y = codecs.bf16_bits_to_f32(codecs.f64_to_bf16_bits(y)).astype(np.float64)
        out = np.zeros((n_tok, y.shape[1])) + (0 if out0 is None else np.asarray(out0, np.float64))
        for r, q in enumerate(np.asarray(row_pair, np.int64)):
            t = q % n_tok if kind == "token_mod" else q // k
            wq = w.reshape(n_tok, k)[t, (q % k + 1) % k] if kind == "slot" else w[q]
            out[t] += wq * y[r]
        return out
    return f


@pytest.mark.parametrize("kind", ["slot", "token_mod", "round_y"])
def test_fused_combine_pins_catch(monkeypatch, kind):
    monkeypatch.setattr(tsw, "swiglu_combine", _fused_mutant(kind))
    results = []
    for t in (tsw.test_fused_combine_matches_pure_python_brute_force,
              tsw.test_fused_combine_k1_unit_weights_is_the_unrounded_ffn,
              tsw.test_fused_combine_invariant_under_row_shuffle_and_skips_bad_ids):
        try:
            t()
            results.append(False)
        except AssertionError:
            results.append(True)
    assert any(results), f"no fused-combine pin caught the {kind} mutant"


# ------------------------------------------------------------------ fp8 grouped GEMM mutants

from oracle import gemm_fp8 as og
from tests import test_oracle_gemm_fp8 as tg


def _product_mutant(kind):
    def f(xq, sx, wq_e, sw_e, col_block, absolute=False):
        m, k = xq.shape
        nb = k // og.BLOCK
        out = np.zeros((m, wq_e.shape[0]))
        for b in range(nb - 1 if kind == "drop_last_block" else nb):
            cols = slice(b * og.BLOCK, (b + 1) * og.BLOCK)
            partial = xq[:, cols] @ wq_e[:, cols].T
            if kind == "transposed_weight_scales":
                col_scale = np.resize(sw_e.T.ravel(), sw_e.size).reshape(sw_e.shape)[:, b]
            else:
                col_scale = sw_e[:, b]
            row_scale = sx[:, (b + 1) % nb] if kind == "row_scale_next_block" else sx[:, b]
            scale = col_scale.astype(np.float64)[col_block][None, :] * \
                row_scale.astype(np.float64)[:, None]
            out += scale * partial
        return out
    return f


@pytest.mark.parametrize("kind", ["transposed_weight_scales", "row_scale_next_block",
                                  "drop_last_block"])
def test_fp8_gemm_pins_catch(monkeypatch, kind):
    monkeypatch.setattr(og, "_expert_product", _product_mutant(kind))
    _fails(tg.test_closed_form_constant_codes_non_square_block_grid)
