"""CPU oracle for MoE routing, dispatch and combine.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, calls or links anything in this package; only the test
suite, the smoke check and the benchmark's CPU-baseline leg use it.  It shares
no code, tables or constants with the HIP kernels.

Two tiers:

* ``brute``  -- pure-Python loops, exact rational arithmetic
  (``fractions.Fraction``) where a sum is taken.  Tiny inputs only.
* the other modules -- numpy, vectorised only where the vectorised form *is*
  the definition (stable argsort, bincount, cumsum, fancy indexing, matmul),
  float64 for floating point.

Sources the definitions follow (cited by page title and section):

* "MLX expert parallelism all_to_all PR 3158" (Facts list): the data-movement
  kernels dispatch_local / combine_weighted_sum / packet_gather /
  packet_scatter, and the dispatch/combine round-trip tests.
* "backends/mlx: runtime MoE expert-sort for decode (issue #20554)"
  (Summary; reviews' correctness notes; author's follow-up "Handler fixes";
  the unsorted-path fix in the CI write-up): the sorted branch flattens
  ``expert_indices [N, top_k]`` before a stable argsort, casts to int32 and
  takes token = order // top_k; the unsorted branch repeats each token top_k
  times with identity ``inv_order``; the switch is ``(M - 1) // sort_cutoff``.
* "One-Sided Expert-Parallel All-to-All for Mixture-of-Experts Inference over
  NVLink" (abstract): rank-major (segment-major) receive buffers that grouped
  GEMMs read in place.

Every function is pinned by tests that do not re-type its formula: brute force
on tiny inputs, closed forms, invariants, library routines and hand-worked
fixtures under ``tests/golden``.  Pins are listed in each module's docstring;
a function without a pin says "parity unpinned" there.
"""
