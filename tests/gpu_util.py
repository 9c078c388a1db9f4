"""Helpers for GPU tests: numpy <-> device tensors and the tolerance checks.

The tolerances follow from the arithmetic:
* fp32 combine output: |g - o| <= 1e-6 * sum_j |w_j y_j| (a k-term fp32 FMA
  chain is within gamma_k * sum|terms|, gamma_8 ~ 4.8e-7);
* bf16 combine output: within one bf16 ulp of the correctly rounded exact
  value, or, where the terms cancel, within the fp32 bound plus half a bf16
  ulp of the result;
* routing weights: 1e-6 relative, with no absolute slack above the fp32
  normal range (W_ATOL = 2^-126, the smallest normal: below it fp32 keeps
  fewer than 24 significant bits); a handful of fp32 roundings plus expf;
* SwiGLU expert FFN (bf16 inputs, fp32 accumulation, h rounded to bf16 on
  both sides): every element within 2e-2 * max(|o|, rms of its row), and each
  expert's relative Frobenius error within 2e-2.  A flipped bf16 rounding of
  one h element moves y by far less; a wrong expert, a dropped K chunk or a
  swapped gate/up moves whole rows by O(1) relative.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import codecs

DEV = "cuda:0"
W_ATOL = 2.0 ** -126          # routing weights: absolute floor only below the fp32 normal range


def to_dev(a: np.ndarray, kind: str | None = None) -> torch.Tensor:
    """float32 -> float32; uint16 bf16 bits -> bfloat16; uint8 -> uint8; int32 -> int32."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def as_f32(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns or float arrays -> float32 values."""
    return codecs.bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_combine(got: np.ndarray, exact: np.ndarray, abs_terms: np.ndarray, out_bf16: bool,
                  what: str = "") -> None:
    """got: device output (float32 or bf16 bits); exact: float64 oracle value;
    abs_terms: float64 sum_j |w_j y_j| per element."""
    if not out_bf16:
        err = np.abs(got.astype(np.float64) - exact)
        bound = 1e-6 * abs_terms
        bad = err > bound
        assert not bad.any(), f"{what}: {bad.sum()} fp32 elements outside 1e-6*sum|terms|, " \
                              f"worst {np.max(err - bound):.3e}"
        return
    g = codecs.bf16_bits_to_f32(got).astype(np.float64)
    r = codecs.bf16_bits_to_f32(codecs.f64_to_bf16_bits(exact)).astype(np.float64)
    one_ulp = np.abs(g - r) <= bf16_ulp(np.maximum(np.abs(g), np.abs(r)))
    cancel_ok = np.abs(g - exact) <= 1e-6 * abs_terms + 0.5 * bf16_ulp(g)
    bad = ~(one_ulp | cancel_ok)
    assert not bad.any(), f"{what}: {bad.sum()} bf16 elements beyond 1 ulp"


def combine_reference(y_rows_f32: np.ndarray, dst_pos: np.ndarray, w: np.ndarray, k: int,
                      tokens=None):
    """(exact value, sum of |terms|) from the oracle for the given tokens."""
    from oracle.combine import combine_f64
    exact = combine_f64(y_rows_f32, dst_pos, w, k, tokens=tokens)
    mag = combine_f64(np.abs(y_rows_f32), dst_pos, np.abs(w), k, tokens=tokens)
    return exact, mag


def check_swiglu(got_bits, ref_bits, experts, what=""):
    g = codecs.bf16_bits_to_f32(got_bits).astype(np.float64)
    o = codecs.bf16_bits_to_f32(ref_bits).astype(np.float64)
    rms = np.sqrt(np.mean(o * o, axis=1, keepdims=True))
    bound = 2e-2 * np.maximum(np.abs(o), rms)
    bad = np.abs(g - o) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements outside 2e-2"
    for e in np.unique(experts):
        sel = experts == e
        rel = np.linalg.norm(g[sel] - o[sel]) / max(np.linalg.norm(o[sel]), 1e-30)
        assert rel <= 2e-2, f"{what}: expert {e} relative error {rel:.3e}"


def check_weights(got: np.ndarray, want: np.ndarray, what: str = "") -> None:
    """Routing weights at 1e-6 relative (absolute floor only for subnormals)."""
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=W_ATOL, err_msg=what)


def tile_rows(offsets, tile: int, rng) -> np.ndarray:
    """Rows to check in a grouped buffer: one random row from every `tile`-row
    tile of every expert (tiles start at the expert's first row, as the
    grouped kernels cut them), plus each non-empty expert's last row."""
    offs = np.asarray(offsets, dtype=np.int64)
    picks = []
    for e in range(offs.size - 1):
        lo, hi = int(offs[e]), int(offs[e + 1])
        for t0 in range(lo, hi, tile):
            picks.append(int(rng.integers(t0, min(t0 + tile, hi))))
        if hi > lo:
            picks.append(hi - 1)
    return np.unique(np.array(picks, dtype=np.int64))


def combine_check_all_tokens(out_dev, y_dev, dst_pos_dev, w_dev, k: int, out_bf16: bool,
                             what: str = "", chunk: int = 512) -> None:
    """Every token of a full-size combine against the float64 oracle, in token
    chunks (the oracle evaluates each token on its own)."""
    y = as_f32(to_np(y_dev))
    dst, w = to_np(dst_pos_dev), to_np(w_dev)
    got = to_np(out_dev)
    n = w.shape[0]
    for t0 in range(0, n, chunk):
        toks = np.arange(t0, min(t0 + chunk, n))
        exact, mag = combine_reference(y, dst, w, k, tokens=toks)
        check_combine(got[toks], exact, mag, out_bf16, what=f"{what} tokens {t0}..")


def per_expert_oracle(fn, experts: np.ndarray, fetch, workers: int = 8):
    """Evaluate an oracle function expert by expert on a thread pool.

    experts: the expert of each selected row; fetch(e) -> the expert's host
    operands; fn(row_indices, local_expert_ids, operands) -> result rows.
    Returns the results stacked in the order of `experts`."""
    from concurrent.futures import ThreadPoolExecutor

    experts = np.asarray(experts)
    uniq = np.unique(experts)

    def one(e):
        sel = np.nonzero(experts == e)[0]
        return sel, fn(sel, np.zeros(sel.size, np.int64), fetch(int(e)))

    from threadpoolctl import threadpool_limits

    out = None
    # one BLAS thread per worker: nested BLAS pools oversubscribe the cores
    with threadpool_limits(1), ThreadPoolExecutor(workers) as pool:
        for sel, res in pool.map(one, uniq):
            if out is None:
                out = np.zeros((experts.size,) + res.shape[1:], dtype=res.dtype)
            out[sel] = res
    return out
