"""Top-k routing oracle (test infrastructure only).

What is computed.  For each token t the router selects the k experts with the
largest fp32 logits and returns ``expert_indices [N, k]`` (the routing output
the MoE gather op consumes: "backends/mlx: runtime MoE expert-sort for decode
(issue #20554)", author's follow-up "Handler fixes", which flattens exactly
this ``[N, top_k]`` array) and fp32 routing weights.

The pages never state the gating function; the workloads served here use
softmax top-k with fp32 weights, renormalised over the selected experts.  The
readings taken:

* selection is on the fp32 logits in the total order (value descending, then
  expert index ascending), with -0.0 == +0.0.  Softmax is strictly monotone,
  so this is the same set as selecting on probabilities, without ties created
  by rounding exp();
* slot 0 holds the best expert, slot k-1 the k-th best;
* ``renormalize``: w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0);
  otherwise w_j = exp(l_j - m) / sum_{e<E} exp(l_e - m), m = max_e l_e;
  computed in float64 and rounded once to float32.

NaN logits are outside the contract.

Pins (tests/test_oracle_route.py): brute force over all experts in pure Python
(``route_topk_brute``) against the numpy form on random, tied and signed-zero
inputs; closed forms -- equal logits give indices 0..k-1 and weights exactly
1/k; k = 2 renormalised gives w_0 = logistic(l_0 - l_1); k = E without
renormalisation equals the full softmax; weights sum to 1 and never increase
with the slot; a hand-worked fixture (tests/golden/route_small.txt).
"""
from __future__ import annotations

import math

import numpy as np


def route_topk(logits: np.ndarray, k: int, renormalize: bool = True):
    """Vectorised oracle.  ``logits`` float32 [N, E] -> (idx int32 [N,k], w float32 [N,k])."""
    l32 = np.asarray(logits, dtype=np.float32)
    n, e = l32.shape
    if not (1 <= k <= e):
        raise ValueError("need 1 <= k <= E")
    l = l32.astype(np.float64) + 0.0          # -0.0 + 0.0 == +0.0: one zero
    # stable sort of -l keeps the lower expert index first among equal values
    order = np.argsort(-l, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(l, order[:, :k], axis=1)
    if renormalize:
        ex = np.exp(sel - sel[:, :1])
        w = ex / ex.sum(axis=1, keepdims=True)
    else:
        m = l.max(axis=1, keepdims=True)
        den = np.exp(l - m).sum(axis=1, keepdims=True)
        w = np.exp(sel - m) / den
    return idx, w.astype(np.float32)


def route_topk_brute(logits, k: int, renormalize: bool = True):
    """Pure-Python oracle for tiny inputs: sort every expert of every token by
    (-value, index), take the first k, and form the weights with math.exp and
    an exactly rounded sum (math.fsum)."""
    rows = [[float(v) for v in row] for row in np.asarray(logits, dtype=np.float32)]
    idx_out, w_out = [], []
    for row in rows:
        e = len(row)
        ranked = sorted(range(e), key=lambda i: (-row[i], i))   # -0.0 == 0.0 in Python
        pick = ranked[:k]
        if renormalize:
            ref = row[pick[0]]
            ex = [math.exp(row[i] - ref) for i in pick]
            den = math.fsum(ex)
        else:
            ref = max(row)
            ex = [math.exp(row[i] - ref) for i in pick]
            den = math.fsum(math.exp(v - ref) for v in row)
        idx_out.append(pick)
        w_out.append([float(np.float32(x / den)) for x in ex])
    return np.array(idx_out, dtype=np.int32).reshape(len(rows), k), \
        np.array(w_out, dtype=np.float32).reshape(len(rows), k)
