"""Oracle for the tree-packed chunkwise gated-delta path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import, call, link or run anything in this package.  The product path
(``chunkwise_linear_attention_gated_amd``) never does, and this package never
imports the product path: the two share no code.  The only common dependency
is the seeded input generator package ``synthetic``, which holds none of the
method's arithmetic.

Contents, each written from the pages (HARTS, arXiv 2608.28158):

* ``oracle.planner``   -- compact tokens (distinct prefixes), map m: S -> C,
  multiplicities q, fork-free segments, the T_pre/T_in minimum-call recursion,
  ASAP round recovery, compact layout, replay row lists and state slots; plus
  an exhaustive minimum-call search for small trees.
* ``oracle.recurrent`` -- the gated delta rule run token by token in float64
  on every expanded root-to-leaf trajectory independently, forward and a
  hand-derived reverse pass (C, OpenMP; ``recurrent.c``).
* ``oracle.chunkwise`` -- float64 chunkwise form of the same rule, and a tree
  execution with bounded replay built on it (used only for self-checks).
* ``oracle.logprob``   -- float64 log-softmax gather from its definition (per position,
  or with each row's log-sum-exp taken once by a library routine), its
  gradient (per-position terms summed into their compact row), occurrence
  counts.
* ``oracle.conv``      -- float64 depthwise causal convolution over each
  trajectory's own tokens (ancestor context), and its gradients.
* ``oracle.attention`` -- float64 softmax attention of every compact row over
  its own root-to-row path (the tree form of the MLA layer's ancestor-KV
  views with bottom-right causal alignment), and its gradients.
* ``oracle.moe``      -- float64 router statistics of compact rows weighted by
  their multiplicities (z-loss, load-balance mass and top-k counts, bias
  update) and the logits' gradient.

Parity status: every function above is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force or a library routine.
"""
