"""Grouped SwiGLU expert FFN oracle (test infrastructure only).

The expert compute that reads the dispatched rows in place: for every row p of
the expert-major buffer with expert e = row_expert[p],

    g = W_gate[e] @ r,  u = W_up[e] @ r          (W_gate, W_up: [E, F, D])
    h = bf16( silu(g) * u ),  silu(a) = a / (1 + exp(-a))
    y[p] = bf16( W_down[e] @ h )                  (W_down: [E, D, F])

Sources: "backends/mlx: runtime MoE expert-sort for decode (issue #20554)"
(first review, schema comments: expert weight matrices are laid out
``[E, out, in]``; follow-up: the sorted flag of gather_mm is a caller's promise
that rows arrive grouped by expert, not a request to sort); "One-Sided
Expert-Parallel All-to-All ... over NVLink" (abstract: grouped GEMMs read the
dispatched buffers in place).  The SwiGLU form and the bf16 rounding of h
between the two products are readings: the pages do not give the
expert's activation.

Arithmetic: float64 on the bf16-valued inputs, h and y rounded once to bf16
(correct rounding from float64).

The same function serves rows in any order, each with its own expert: the
per-row expert ids of gather_mm on the unsorted decode layout ("backends/mlx:
runtime MoE expert-sort for decode (issue #20554)", Summary), and the batched
expert FFN planned for decode in "MLX expert parallelism all_to_all PR 3158"
(Facts list).

swiglu_combine is the weighted top-k sum taken straight from the FFN result,
the zero-copy combine that the same MLX PR planned (Facts list): out[t] =
out0[t] + sum_j w_tj * y(t, j), with y never rounded to bf16 -- our reading of
a combine fused into the down product, whose accumulator is fp32.

Pins (tests/test_oracle_swiglu.py): a pure-Python brute force (math.fsum dot
products) on a tiny case; silu closed forms (silu(0) = 0, odd-part identity
silu(a) - silu(-a) = a); layout invariance -- the output for pair (t, j) does
not depend on where dispatch put its row; empty experts produce no rows; the
fused combine against a pure-Python brute force (pairs looked up by scanning
the rows), its k = 1 / unit-weight special case, and its invariance under a
shuffle of the rows.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import bf16_bits_to_f32, f64_to_bf16_bits


def silu(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(-a))


def _hidden_bits(x_f64: np.ndarray, wg_bf16: np.ndarray, wu_bf16: np.ndarray) -> np.ndarray:
    """h = bf16(silu(W_gate x) * (W_up x)) for the rows of x (one expert)."""
    wg = bf16_bits_to_f32(wg_bf16).astype(np.float64)
    wu = bf16_bits_to_f32(wu_bf16).astype(np.float64)
    return f64_to_bf16_bits(silu(x_f64 @ wg.T) * (x_f64 @ wu.T))


def swiglu_hidden(rows_bf16: np.ndarray, experts: np.ndarray, w_gate_bf16, w_up_bf16) -> np.ndarray:
    """The hidden activation h [M, F] (uint16 bf16 bits) between the two
    products, for rows with their experts; rows whose expert lies outside
    [0, E) give zeros.  The same h that swiglu_rows multiplies by W_down."""
    r = bf16_bits_to_f32(rows_bf16).astype(np.float64)
    experts = np.asarray(experts, dtype=np.int64)
    w_gate = np.asarray(w_gate_bf16)
    out = np.zeros((r.shape[0], w_gate.shape[1]), dtype=np.uint16)
    for e in np.unique(experts):
        if e < 0 or e >= w_gate.shape[0]:
            continue
        sel = np.nonzero(experts == e)[0]
        out[sel] = _hidden_bits(r[sel], w_gate[e], w_up_bf16[e])
    return out


def swiglu_rows_f64(rows_bf16: np.ndarray, experts: np.ndarray, w_gate_bf16, w_up_bf16,
                    w_down_bf16) -> np.ndarray:
    """float64 [M, D] value of y before its final rounding (h is rounded to
    bf16 as in the definition).  Rows whose expert lies outside [0, E) give 0
    (they take no part)."""
    r = bf16_bits_to_f32(rows_bf16).astype(np.float64)
    experts = np.asarray(experts, dtype=np.int64)
    n_exp = np.asarray(w_gate_bf16).shape[0]
    out = np.zeros(r.shape, dtype=np.float64)
    for e in np.unique(experts):
        if e < 0 or e >= n_exp:
            continue
        sel = np.nonzero(experts == e)[0]
        h = bf16_bits_to_f32(_hidden_bits(r[sel], w_gate_bf16[e], w_up_bf16[e])).astype(np.float64)
        wd = bf16_bits_to_f32(w_down_bf16[e]).astype(np.float64)
        out[sel] = h @ wd.T
    return out


def swiglu_rows(rows_bf16: np.ndarray, experts: np.ndarray, w_gate_bf16, w_up_bf16,
                w_down_bf16) -> np.ndarray:
    """Evaluate the expert FFN on selected rows.

    rows_bf16 uint16 [M, D]; experts int [M]; weights uint16 bit patterns
    (indexable by expert: [E, F, D], [E, F, D], [E, D, F]).  Returns y as
    uint16 bf16 bit patterns [M, D]."""
    return f64_to_bf16_bits(swiglu_rows_f64(rows_bf16, experts, w_gate_bf16, w_up_bf16,
                                            w_down_bf16))


def swiglu_combine(rows_bf16, experts, row_pair, topk_w, k: int, w_gate_bf16, w_up_bf16,
                   w_down_bf16, out0=None) -> np.ndarray:
    """The combine fused into the expert FFN (zero-copy combine): for every
    token t,

        out[t] = out0[t] + sum_j topk_w[t, j] * y(t, j)

    where y(t, j) is the FFN output, before any rounding of y, of the row r
    holding pair q = t*k + j (row_pair[r] == q) computed with expert
    experts[r].  Rows with an expert outside [0, E) add nothing.  float64
    [N, D]; N = len(topk_w) // k (topk_w flattened over [N, k])."""
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64).reshape(-1)
    n_tok = w.size // k
    y = swiglu_rows_f64(rows_bf16, experts, w_gate_bf16, w_up_bf16, w_down_bf16)
    out = np.zeros((n_tok, y.shape[1]), dtype=np.float64)
    if out0 is not None:
        out += np.asarray(out0, dtype=np.float64)
    q = np.asarray(row_pair, dtype=np.int64)
    for r in range(q.size):           # each row adds its term to its token
        out[q[r] // k] += w[q[r]] * y[r]
    return out


def grouped_swiglu(rows_bf16, expert_offsets, w_gate_bf16, w_up_bf16, w_down_bf16):
    """The whole expert-major buffer: expert e owns rows
    [expert_offsets[e], expert_offsets[e+1])."""
    offs = np.asarray(expert_offsets, dtype=np.int64)
    experts = np.repeat(np.arange(offs.size - 1), np.diff(offs))
    return swiglu_rows(rows_bf16, experts, w_gate_bf16, w_up_bf16, w_down_bf16)


def swiglu_brute(row, wg, wu, wd):
    """Pure-Python single row, float weights as nested lists; returns the
    float64 value of y before its final bf16 rounding, with h rounded to bf16
    through a Python re-implementation of RNE on the float32 grid."""
    f = len(wg)
    g = [math.fsum(a * b for a, b in zip(wg[i], row)) for i in range(f)]
    u = [math.fsum(a * b for a, b in zip(wu[i], row)) for i in range(f)]
    h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    hb = [_bf16_round_py(v) for v in h]
    return [math.fsum(a * b for a, b in zip(wd[i], hb)) for i in range(len(wd))]


def _bf16_round_py(v: float) -> float:
    """RNE of a Python float to bfloat16, by scaling: bf16 keeps 8 significant
    bits, so round v * 2**(7 - e) to an integer with ties to even."""
    if v == 0.0 or not math.isfinite(v):
        return v
    m, e = math.frexp(abs(v))          # abs(v) = m * 2**e, 0.5 <= m < 1
    e = max(e, -125)                   # subnormal spacing below the bf16 normal range
    scaled = abs(v) * 2.0 ** (8 - e)   # 8 significant bits above the point
    q = round(scaled)                  # Python round(): ties to even
    return math.copysign(q * 2.0 ** (e - 8), v)
