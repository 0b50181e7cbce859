"""CPU oracle for the Mesh-Attention tile hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the test-suite, the smoke check and the benchmark's CPU-baseline leg use it.

The oracle is written from the definitions on the pages, in float64 numpy,
with no blocking, no online softmax and no fusion:

* ``block_list_ref``  - which (Q partition, KV partition) blocks one GPU of an
  R x C mesh owns, in KV-partition-rotation order, and each block's causal
  class (full / diagonal / skipped), found by brute force over token positions.
* ``attention_ref`` / ``tile_rows_ref`` - exact two-pass softmax attention of
  query rows over an arbitrary set of keys, returning the output and the
  natural-log log-sum-exp of the scaled scores.
* ``lse_merge_ref``  - the log-sum-exp weighted combination of partial
  (output, lse) pairs.
* ``greedy_plan_ref`` / ``optimal_makespan_ref`` - the greedy schedule of
  transfers and block computations of one mesh GPU, and the exhaustive
  optimum of the same step model on tiny meshes.
* ``attention_bwd_ref`` / ``tile_bwd_ref`` / ``bwd_delta_ref`` - the gradients
  of attention (dQ, dK, dV) split into the share of one tile's visible pairs,
  given the rows' final lse and D = rowsum(dO * O).

Every function here is pinned by CPU tests to something other than itself
(library routines, closed forms, invariants, brute force); see the test files
named ``test_oracle_*.py``.
"""

from .block_list import FULL, DIAG, SKIP, block_list_ref, mesh_tile_sets_ref
from .attention import attention_ref, tile_rows_ref, tile_positions_ref
from .merge import lse_merge_ref
from .backward import attention_bwd_ref, bwd_delta_ref, full_grads_ref, tile_bwd_ref
from .schedule import greedy_plan_ref, optimal_makespan_ref, plan_makespan_ref

__all__ = [
    "FULL", "DIAG", "SKIP",
    "block_list_ref", "mesh_tile_sets_ref",
    "attention_ref", "tile_rows_ref", "tile_positions_ref",
    "lse_merge_ref",
    "attention_bwd_ref", "bwd_delta_ref", "full_grads_ref", "tile_bwd_ref",
    "greedy_plan_ref", "optimal_makespan_ref", "plan_makespan_ref",
]
