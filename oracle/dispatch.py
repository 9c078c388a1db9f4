"""Dispatch oracle: counts, offsets, the stable permutation and the row copy
(test infrastructure only).

Notation: N tokens, k experts per token, E experts, G segments (contiguous
groups of E/G experts), NK = N*k routed pairs, pair q = t*k + j.

Sources.
* "backends/mlx: runtime MoE expert-sort for decode (issue #20554)":
  - author's follow-up "Handler fixes": the sorted branch flattens
    ``expert_indices [N, top_k]`` to ``[N*top_k]`` before the argsort, casts
    the order to int32, and recovers the token as order // top_k;
  - the CI write-up ("What this tip is"): on the unsorted branch
    ``inv_order`` is the identity ``arange(N*top_k)`` and the input rows are
    ``x.repeat_interleave(top_k)``;
  - the reviews' correctness notes: the switch is ``cond = (M-1) //
    sort_cutoff``, M <= cutoff -> unsorted, M > cutoff -> sorted; both
    branches emit the same N*top_k-row shape.
* "MLX expert parallelism all_to_all PR 3158" (Facts): dispatch_local /
  packet_gather / packet_scatter move O(N*D) rows; dispatch/combine are tested
  by round trip.
* "One-Sided Expert-Parallel All-to-All ... over NVLink" (abstract): tokens
  land in rank-major blocks that grouped GEMMs read in place -- read here as
  segment-major blocks, segment g = experts [g*E/G, (g+1)*E/G).

Readings: the argsort is stable (ties keep the flattened
pair order t*k + j); sorted mode buckets by expert; unsorted mode buckets by
segment (G = 1: one bucket, so the permutation is the identity); no capacity
limit and no padding between blocks; ``dst_pos`` plays the role of
``inv_order`` (indexed by pair), ``src_pair`` is the argsort order (indexed by
row), ``row_expert[p]`` is the expert of row p.

Pins (tests/test_oracle_dispatch.py): O(NK^2) brute force ``permutation_brute``
against the argsort form; counts against a Python Counter; sum(counts) == NK;
``src_pair`` is a permutation and ``dst_pos`` its inverse; identity in
unsorted G=1 mode; sorted G=8 equals sorted G=1; rows equal x at
src_pair // k; hand-worked fixture tests/golden/dispatch_small.txt.
"""
from __future__ import annotations

import numpy as np


def resolve_sorted(sort: int, n_tokens: int, sort_cutoff: int) -> bool:
    """Runtime sort switch.  sort = 1 forces sorted, 0 forces unsorted, -1 asks
    for the switch: sorted iff (N - 1) // cutoff >= 1, i.e. N > cutoff.  A
    cutoff <= 0 means "always sort" (the divide-by-zero guard's reading)."""
    if sort == 1:
        return True
    if sort == 0:
        return False
    if sort != -1:
        raise ValueError("sort must be -1, 0 or 1")
    if sort_cutoff <= 0:
        return True
    return (n_tokens - 1) // sort_cutoff >= 1 if n_tokens > 0 else False


def expert_counts(idx: np.ndarray, n_experts: int) -> np.ndarray:
    return np.bincount(np.asarray(idx).ravel(), minlength=n_experts).astype(np.int32)


def expert_offsets(counts: np.ndarray) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def segment_offsets(offsets: np.ndarray, n_experts: int, n_segments: int) -> np.ndarray:
    """Start of each segment's block.  Segments are contiguous expert ranges,
    so a segment's rows start where its first expert's rows start; the same
    holds in unsorted mode, where the block of segment g holds exactly the
    pairs routed to its experts."""
    step = n_experts // n_segments
    return np.asarray(offsets)[::step].astype(np.int32)


def bucket_keys(idx: np.ndarray, n_experts: int, n_segments: int, sorted_: bool) -> np.ndarray:
    flat = np.asarray(idx, dtype=np.int64).ravel()
    return flat if sorted_ else flat // (n_experts // n_segments)


def permutation(idx: np.ndarray, n_experts: int, n_segments: int, sorted_: bool):
    """-> (src_pair [NK], dst_pos [NK], row_expert [NK]) int32."""
    flat = np.asarray(idx, dtype=np.int64).ravel()
    key = bucket_keys(idx, n_experts, n_segments, sorted_)
    src_pair = np.argsort(key, kind="stable")
    dst_pos = np.empty_like(src_pair)
    dst_pos[src_pair] = np.arange(src_pair.size)
    row_expert = flat[src_pair]
    return src_pair.astype(np.int32), dst_pos.astype(np.int32), row_expert.astype(np.int32)


def permutation_brute(idx, n_experts: int, n_segments: int, sorted_: bool):
    """Pure-Python definition for tiny inputs: the position of pair q is the
    start of its bucket plus the number of earlier pairs (in flattened order)
    with the same bucket key."""
    flat = [int(v) for v in np.asarray(idx).ravel()]
    step = n_experts // n_segments
    key = [v if sorted_ else v // step for v in flat]
    n_buckets = n_experts if sorted_ else n_segments
    count = [0] * n_buckets
    for kk in key:
        count[kk] += 1
    start = [0] * n_buckets
    for b in range(1, n_buckets):
        start[b] = start[b - 1] + count[b - 1]
    dst = []
    for q, kk in enumerate(key):
        dst.append(start[kk] + sum(1 for q2 in range(q) if key[q2] == kk))
    src = [0] * len(flat)
    for q, p in enumerate(dst):
        src[p] = q
    rexp = [flat[src[p]] for p in range(len(flat))]
    return (np.array(src, dtype=np.int32), np.array(dst, dtype=np.int32),
            np.array(rexp, dtype=np.int32))


def gather_rows(x: np.ndarray, src_pair: np.ndarray, k: int) -> np.ndarray:
    """rows[p] = x[src_pair[p] // k] -- the gather form (packet_gather).
    Works on any dtype; bit patterns are copied unchanged."""
    return np.asarray(x)[np.asarray(src_pair, dtype=np.int64) // k]


def scatter_rows(x: np.ndarray, dst_pos: np.ndarray, k: int) -> np.ndarray:
    """rows[dst_pos[t*k+j]] = x[t] -- the scatter form (packet_scatter).
    Written as an explicit loop over pairs so that it is an independent check
    of ``gather_rows``."""
    x = np.asarray(x)
    dst = np.asarray(dst_pos, dtype=np.int64)
    rows = np.empty((dst.size,) + x.shape[1:], dtype=x.dtype)
    for q in range(dst.size):
        rows[dst[q]] = x[q // k]
    return rows


def dispatch(idx, n_experts: int, n_segments: int, sorted_: bool, x=None, x_scales=None):
    """Everything the dispatch call produces, as a dict of numpy arrays."""
    idx = np.asarray(idx)
    k = idx.shape[1] if idx.ndim == 2 else 1
    counts = expert_counts(idx, n_experts)
    offs = expert_offsets(counts)
    segs = segment_offsets(offs, n_experts, n_segments)
    src, dst, rexp = permutation(idx, n_experts, n_segments, sorted_)
    out = dict(expert_counts=counts, expert_offsets=offs, segment_offsets=segs,
               src_pair=src, dst_pos=dst, row_expert=rexp)
    if x is not None:
        out["rows"] = gather_rows(x, src, k)
    if x_scales is not None:
        out["row_scales"] = gather_rows(x_scales, src, k)
    return out
