"""Combine oracle: weighted top-k gather-sum back to token order (test
infrastructure only).

    out[t, i] = sum_{j<k} w[t, j] * y[dst_pos[t*k + j], i]

"MLX expert parallelism all_to_all PR 3158" (Facts) names the kernel
combine_weighted_sum; "backends/mlx: runtime MoE expert-sort for decode (issue
#20554)" (CI write-up) has ``moe_scatter_outputs`` undo the input permutation
with ``inv_order`` before the weighted sum -- here ``dst_pos`` is that inverse
map, so the unscatter and the sum are one step.  The weight multiplies the
expert output (it is applied after the expert).

The oracle sums exactly and rounds once:
* ``combine_exact_brute``: Fraction arithmetic, then RNE to the output format;
* ``combine_f64``: float64 products (exact: 24-bit by 24-bit significands fit
  in 53 bits) summed in float64 -- relative error below k * 2**-53 of
  sum |terms|, negligible beside the tolerances used -- returned unrounded so
  that the tests can apply the output format's rounding and tolerance.

Tolerances (the GPU tests apply them): fp32 output within
1e-6 * sum_j |w_j * y_j| per element; bf16 output within one bf16 ulp of the
correctly rounded exact value.

Pins (tests/test_oracle_combine.py): Fraction brute force vs float64 form;
identity experts with renormalised weights reproduce x within 2k ulp;
one-hot weights return y rows bit-exactly (round trip of dispatch then
combine); doubling the weights doubles the output exactly; hand-worked
fixture tests/golden/combine_small.txt.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .codecs import fraction_to_bf16_bits, fraction_to_f32


def combine_f64(y: np.ndarray, dst_pos: np.ndarray, w: np.ndarray, k: int,
                tokens=None) -> np.ndarray:
    """float64 [N or len(tokens), D] value of the weighted sum (unrounded).

    ``y`` is float32/float64 [NK, D] (decode bf16 first); ``tokens`` selects a
    subset of tokens to evaluate one by one (for full-size sampled checks)."""
    y = np.asarray(y)
    dst = np.asarray(dst_pos, dtype=np.int64).reshape(-1, k)
    w = np.asarray(w, dtype=np.float32).astype(np.float64).reshape(-1, k)
    ts = np.arange(dst.shape[0]) if tokens is None else np.asarray(tokens)
    out = np.zeros((ts.size, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[ts, j:j + 1] * y[dst[ts, j]].astype(np.float64)
    return out


def combine_exact_brute(y, dst_pos, w, k: int, out_format: str):
    """Pure-Python exact rational sum for tiny inputs, rounded once.

    out_format 'f32' -> float32 array; 'bf16' -> uint16 bit patterns."""
    y = np.asarray(y, dtype=np.float64)
    dst = [int(v) for v in np.asarray(dst_pos).ravel()]
    wf = [float(v) for v in np.asarray(w, dtype=np.float32).ravel()]
    n = len(dst) // k
    d = y.shape[1]
    res = []
    for t in range(n):
        row = []
        for i in range(d):
            s = Fraction(0)
            for j in range(k):
                s += Fraction(wf[t * k + j]) * Fraction(float(y[dst[t * k + j], i]))
            row.append(fraction_to_f32(s) if out_format == "f32" else fraction_to_bf16_bits(s))
        res.append(row)
    if out_format == "f32":
        return np.array(res, dtype=np.float32).reshape(n, d)
    return np.array(res, dtype=np.uint16).reshape(n, d)
