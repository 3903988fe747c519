"""Seeded synthetic inputs shared by the oracle side and the device side.

This package draws random numbers and lays out rollout-tree structures; it
holds none of the method's arithmetic (no prefix merging, no planning, no
gated-delta math, no softmax).  Both sides receive exactly the same values.

* ``synthetic.trees``   -- rollout trees given as fork-free segments, and the
  trajectories (token id sequences) they expand to.
* ``synthetic.tensors`` -- per-node q/k/v/g/beta/dO features, bf16 rounding,
  and the compact-row log-prob workload (multiplicities, labels, logits).
"""
from . import trees, tensors  # noqa: F401
