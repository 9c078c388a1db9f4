"""fp8 block-scaled grouped expert GEMM (test infrastructure only).

"One-Sided Expert-Parallel All-to-All for Mixture-of-Experts Inference over
NVLink" (abstract): the dispatch is agnostic to the activation quantisation
format and the grouped GEMMs read the received (rank-major) buffers in place.
The consumer defined here takes the dispatched fp8 rows exactly as the
dispatch leaves them: E4M3FN codes with one float32 scale per 128 elements of
a row (the segment-major workload's format), grouped by expert
(``offsets[e] .. offsets[e+1]``), and expert weights stored the same way at a
coarser grain: E4M3FN codes ``w_q [E, N, K]`` with one float32 scale per
128 x 128 block, ``w_scales [E, N/128, K/128]``.  For a row p of expert e:

    y[p, n] = bf16( sum_b  sx[p, b] * sw[e, n // 128, b]
                         * sum_{k in block b} q(rows[p, k]) * q(w[e, n, k]) )

with b over the K/128 blocks of 128.  The inner sums are exact in float64
(products of two E4M3 values have 8 significant bits, 128 of them need at most
43 bits); the scaled sum over blocks is float64; the result is rounded once
to bfloat16.

``gemm_fp8_magnitude`` gives the same sum with every term replaced by its
absolute value: the scale of the rounding error of any finite-precision
accumulation of these terms.

Pins (tests/test_oracle_gemm_fp8.py): a closed form for constant codes and
power-of-two block scales on a non-square block grid (a transposed scale
index fails it); exact rational brute force on a tiny case; torch's own
float8 decode and a float64 matmul as an independent route (also for a
subset of output columns spread over several 128-column blocks); the
per-expert weight selection through ragged offsets, including an empty
expert.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .codecs import f64_to_bf16_bits, fp8_bits_to_f64

BLOCK = 128


def _check(rows_q, row_scales, w_q, w_scales):
    r, k = rows_q.shape
    e, n, k2 = w_q.shape
    if k != k2 or k % BLOCK or n % BLOCK:
        raise ValueError("K must match and K, N must be multiples of 128")
    if row_scales.shape != (r, k // BLOCK) or w_scales.shape != (e, n // BLOCK, k // BLOCK):
        raise ValueError("scale shapes")


def _expert_product(xq, sx, wq_e, sw_e, col_block, absolute=False):
    """xq [m, K] and wq_e [C, K] (C output columns) as float64 values, sx
    [m, K/128], sw_e [N/128, K/128], col_block [C]: the 128-column block of
    each output column (n // 128) -> float64 [m, C]."""
    m, k = xq.shape
    out = np.zeros((m, wq_e.shape[0]))
    for b in range(k // BLOCK):
        ks = slice(b * BLOCK, (b + 1) * BLOCK)
        a, w = xq[:, ks], wq_e[:, ks]
        if absolute:
            a, w = np.abs(a), np.abs(w)
        partial = a @ w.T                                       # exact in float64
        scale = sw_e[col_block, b].astype(np.float64)[None, :] * \
            sx[:, b].astype(np.float64)[:, None]
        out += (np.abs(scale) if absolute else scale) * partial
    return out


def gemm_fp8_rows(rows_q, row_scales, experts, w_q, w_scales, absolute=False, cols=None):
    """float64 y for the given rows; ``experts[i]`` is the expert of row i.

    ``cols`` (optional) lists the output columns n to evaluate, in the order
    of the result's columns; by default every column.  Each element is the
    same sum either way -- only fewer of them are formed, and only the weight
    rows w[e, n] they need are decoded."""
    rows_q = np.asarray(rows_q, np.uint8)
    row_scales = np.asarray(row_scales, np.float32)
    w_q = np.asarray(w_q, np.uint8)
    w_scales = np.asarray(w_scales, np.float32)
    _check(rows_q, row_scales, w_q, w_scales)
    experts = np.asarray(experts, np.int64)
    cols = np.arange(w_q.shape[1]) if cols is None else np.asarray(cols, np.int64)
    out = np.zeros((rows_q.shape[0], cols.size))
    xq = fp8_bits_to_f64(rows_q)
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        out[sel] = _expert_product(xq[sel], row_scales[sel], fp8_bits_to_f64(w_q[e][cols]),
                                   w_scales[e], cols // BLOCK, absolute)
    return out


def grouped_gemm_fp8(rows_q, row_scales, offsets, w_q, w_scales):
    """Rows grouped by expert through ``offsets [E+1]`` -> (y bf16 bits
    [R, N], y float64 [R, N]).  Rows outside [offsets[0], offsets[E]) are
    left at zero."""
    offsets = np.asarray(offsets, np.int64)
    r = np.asarray(rows_q).shape[0]
    experts = np.full(r, -1, np.int64)
    for e in range(len(offsets) - 1):
        experts[offsets[e]:offsets[e + 1]] = e
    y = np.zeros((r, np.asarray(w_q).shape[1]))
    sel = np.nonzero(experts >= 0)[0]
    if sel.size:
        y[sel] = gemm_fp8_rows(np.asarray(rows_q)[sel], np.asarray(row_scales)[sel], experts[sel],
                               w_q, w_scales)
    return f64_to_bf16_bits(y), y


def gemm_fp8_magnitude(rows_q, row_scales, experts, w_q, w_scales, cols=None):
    """Sum of the absolute values of every term of y (same rows and columns as
    ``gemm_fp8_rows``)."""
    return gemm_fp8_rows(rows_q, row_scales, experts, w_q, w_scales, absolute=True, cols=cols)


def gemm_fp8_brute(rows_q, row_scales, experts, w_q, w_scales):
    """Exact rational value of every output (pure Python, tiny inputs)."""
    r, k = np.asarray(rows_q).shape
    n = np.asarray(w_q).shape[1]
    xq = fp8_bits_to_f64(np.asarray(rows_q, np.uint8))
    out = [[Fraction(0)] * n for _ in range(r)]
    for p in range(r):
        e = int(experts[p])
        wq = fp8_bits_to_f64(np.asarray(w_q, np.uint8)[e])
        for j in range(n):
            acc = Fraction(0)
            for b in range(k // BLOCK):
                s = Fraction(float(row_scales[p][b])) * Fraction(float(w_scales[e][j // BLOCK][b]))
                part = Fraction(0)
                for kk in range(b * BLOCK, (b + 1) * BLOCK):
                    part += Fraction(float(xq[p, kk])) * Fraction(float(wq[j, kk]))
                acc += s * part
            out[p][j] = acc
    return out
