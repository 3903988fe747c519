"""Rollout trees for tests and benchmarks, described by fork-free segments.

A tree is a list of segments.  Segment ``j`` has a parent segment (or -1 for a
root) and a token count; it starts at absolute position ``start[j]`` equal to
the end of its parent.  Every generated token is a *node*: node ids are
assigned segment by segment in creation order, so ``node_base[j] + i`` is the
node of the i-th token of segment ``j``.  A trajectory is the token path from a
root to the end of a leaf segment (or, for the degenerate cases, to any chosen
position); its semantic positions carry the node ids of the tokens they
traverse, which is how per-node features reach both the oracle and the device.

Token ids are random, with the constraint that children of one segment (and
the roots of a forest) get pairwise distinct first tokens, increasing in the
order the children are listed.  A prefix trie over
the emitted trajectories therefore reproduces the generated tree exactly.

Workloads (sizes are those of the HARTS rollout-tree evaluation, described on
the thelatestinai page of arXiv 2608.28158 and in the paper's rollout-tree
setting; the trees themselves are synthetic stand-ins for the SWE-bench /
tau^3-Bench rollout trees, which are not available here):

* :func:`tiny_tree` -- the 40-token root / 37+29 children / 18-token grandchild
  example in its two readings ``"G"`` and ``"D"``.
* :func:`random_rollout_tree` -- 16384-token root, 64 leaves, fan-out 2..4,
  fork offsets uniform over current tokens and never chunk-aligned, new leaf
  lengths log-uniform in [64, 4096].
* :func:`figure1_tree`, :func:`figure2_tree`, :func:`figureC1_tree` -- token
  counts chosen to realise the call assignments drawn in Figures 1, 2 and C.1.
* :func:`random_small_tree` -- a few segments with small lengths, for brute
  force planner checks.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

DEFAULT_VOCAB = 131072


@dataclass
class GenTree:
    parent: List[int]
    length: List[int]
    # optional extra trajectories ending inside the tree: (segment, tokens taken from it)
    extra_ends: List[Tuple[int, int]] = field(default_factory=list)
    # trajectory indices (into the leaf list) emitted twice
    duplicates: List[int] = field(default_factory=list)

    # ---- derived by finalize() ----
    start: Optional[np.ndarray] = None
    node_base: Optional[np.ndarray] = None
    n_nodes: int = 0
    seg_tokens: Optional[List[np.ndarray]] = None
    tokens: Optional[np.ndarray] = None        # int32 [S] concatenated trajectories
    offsets: Optional[np.ndarray] = None       # int64 [n_traj + 1]
    node_of_pos: Optional[np.ndarray] = None   # int64 [S]
    traj_leaf: Optional[List[Tuple[int, int]]] = None  # (segment, tokens taken) per trajectory

    @property
    def n_traj(self) -> int:
        return len(self.offsets) - 1

    @property
    def S(self) -> int:
        return int(self.offsets[-1])

    def children(self) -> List[List[int]]:
        ch: List[List[int]] = [[] for _ in self.parent]
        for j, p in enumerate(self.parent):
            if p >= 0:
                ch[p].append(j)
        return ch

    def finalize(self, seed: int = 0, vocab: int = DEFAULT_VOCAB, shuffle: bool = True) -> "GenTree":
        """Assign positions, node ids and token ids; emit trajectories."""
        rng = np.random.default_rng(np.random.PCG64([seed, 0x7733]))
        n = len(self.parent)
        order = _topo(self.parent)
        start = np.zeros(n, dtype=np.int64)
        for j in order:
            p = self.parent[j]
            start[j] = 0 if p < 0 else start[p] + self.length[p]
        node_base = np.zeros(n, dtype=np.int64)
        acc = 0
        for j in range(n):
            node_base[j] = acc
            acc += self.length[j]
        seg_tokens = [rng.integers(1, vocab, size=self.length[j]).astype(np.int32) for j in range(n)]
        # distinct first tokens among siblings (and among roots)
        ch = self.children()
        groups = [[j for j in range(n) if self.parent[j] < 0]] + [c for c in ch if len(c) > 1]
        for grp in groups:
            # pairwise distinct first tokens, increasing in listing order, so the
            # first-token order of siblings is the order they are listed in
            firsts = np.sort(rng.choice(np.arange(1, vocab), size=len(grp), replace=False))
            for j, t in zip(grp, firsts):
                if self.length[j] > 0:
                    seg_tokens[j][0] = int(t)
        self.start, self.node_base, self.n_nodes, self.seg_tokens = start, node_base, acc, seg_tokens
        leaves = [(j, self.length[j]) for j in range(n) if not ch[j]]
        ends = leaves + list(self.extra_ends) + [leaves[i] for i in self.duplicates]
        if shuffle:
            perm = rng.permutation(len(ends))
            ends = [ends[i] for i in perm]
        toks, nodes, offs = [], [], [0]
        for (seg, take) in ends:
            path = []
            j = seg
            while j >= 0:
                path.append(j)
                j = self.parent[j]
            path.reverse()
            t_parts, n_parts = [], []
            for j in path:
                cnt = take if j == seg else self.length[j]
                t_parts.append(seg_tokens[j][:cnt])
                n_parts.append(node_base[j] + np.arange(cnt, dtype=np.int64))
            t = np.concatenate(t_parts)
            toks.append(t)
            nodes.append(np.concatenate(n_parts))
            offs.append(offs[-1] + len(t))
        self.tokens = np.concatenate(toks).astype(np.int32)
        self.node_of_pos = np.concatenate(nodes).astype(np.int64)
        self.offsets = np.asarray(offs, dtype=np.int64)
        self.traj_leaf = ends
        return self

    def trajectory(self, i: int) -> np.ndarray:
        return self.tokens[self.offsets[i]:self.offsets[i + 1]]

    def trajectory_nodes(self, i: int) -> np.ndarray:
        return self.node_of_pos[self.offsets[i]:self.offsets[i + 1]]


def _topo(parent: Sequence[int]) -> List[int]:
    n = len(parent)
    depth = [-1] * n

    def d(j):
        if depth[j] >= 0:
            return depth[j]
        chain = []
        while j >= 0 and depth[j] < 0:
            chain.append(j)
            j = parent[j]
        base = -1 if j < 0 else depth[j]
        for k in reversed(chain):
            base += 1
            depth[k] = base
        return depth[chain[0]]

    for j in range(n):
        d(j)
    return sorted(range(n), key=lambda j: depth[j])


def tiny_tree(reading: str = "G", seed: int = 0) -> GenTree:
    """The small CPU-checkable tree (H=2, d=16, B=16 workload).

    Its description -- a 40-token root forking at offset 23 into children of 37
    and 29 tokens, with a grandchild fork at offset 9 of 18 tokens -- admits no
    literal reading that has both 3 leaves and ~150 compact tokens.  Two
    readings are provided:

    * ``"G"`` uses every number: root path [0,40) forks at 23, so the shared
      part is [0,23) with children: the root remainder [23,40), a 37-token child
      [23,60) and a 29-token child [23,52).  The 37-token child forks at its
      offset 9 (absolute 32) into its remainder [32,60) and an 18-token
      grandchild [32,50).  4 leaves, 124 compact tokens.
    * ``"D"`` has 3 leaves: root [0,40) with children of 37 and 29 tokens at 40;
      the 37-token child forks at its offset 9 into [49,77) and an 18-token
      grandchild [49,67).  124 compact tokens.
    """
    if reading == "G":
        # 0: [0,23) 1: root rest [23,40) 2: C1 head [23,32) 3: C2 [23,52) 4: C1 rest [32,60) 5: G [32,50)
        t = GenTree(parent=[-1, 0, 0, 0, 2, 2], length=[23, 17, 9, 29, 28, 18])
    elif reading == "D":
        # 0: root [0,40) 1: C1 head [40,49) 2: C2 [40,69) 3: C1 rest [49,77) 4: G [49,67)
        t = GenTree(parent=[-1, 0, 0, 1, 1], length=[40, 9, 29, 28, 18])
    else:
        raise ValueError(reading)
    return t.finalize(seed=seed)


def figure1_tree(seed: int = 0) -> GenTree:
    """Figure 1 (thelatestinai page): A -> {B, C}, B -> {D, E}; call 1 runs
    [A,B,D], call 2 runs [C] and [E] (B=64).  Token counts are ours: A=100,
    B=10, C=20, D=30, E=25 (A crosses the boundary at 64, so the side branches
    wait one call)."""
    return GenTree(parent=[-1, 0, 0, 1, 1], length=[100, 10, 20, 30, 25]).finalize(seed=seed)


def figure2_tree(seed: int = 0) -> GenTree:
    """Figure 2: v0 -> {v1, v2}, v1 -> {v3, v4}; round 1 packs v0->v1->v3 plus
    replay-started v2, round 2 runs replay-started v4 (B=64).  Token counts are
    ours: v0=40 (no boundary crossed, so v2 starts with the zero state in round
    1), v1=100 (crosses 64 and 128), v2=30, v3=50, v4=20."""
    return GenTree(parent=[-1, 0, 0, 1, 1], length=[40, 100, 30, 50, 20]).finalize(seed=seed)


def figureC1_tree(seed: int = 0) -> GenTree:
    """Figure C.1: shared path P0|P1 (one 84-token segment: P0 = 64 tokens,
    P1 = 20) branches into A, B, C; A continues in round 1, B and C start in
    round 2 from the boundary state after P0 and replay P1 (B=64)."""
    return GenTree(parent=[-1, 0, 0, 0], length=[84, 40, 30, 25]).finalize(seed=seed)


def random_rollout_tree(seed: int = 0, root_len: int = 16384, n_leaves: int = 64,
                        chunk: int = 64, min_leaf: int = 64, max_leaf: int = 4096) -> GenTree:
    """Random rollout tree (the 64-leaf, 16384-token-root workload).

    Start from one root leaf of ``root_len`` tokens.  Until there are
    ``n_leaves`` leaves: pick a fork position uniformly over all current tokens
    (a segment with probability proportional to its length, then an offset
    uniform in [1, len-1] whose absolute position is not a multiple of
    ``chunk``), split that segment there, and attach f-1 new leaves, f uniform
    in {2,3,4} clipped so the leaf count never exceeds ``n_leaves``; each new
    leaf has round(exp(U[ln min_leaf, ln max_leaf])) tokens.
    """
    rng = np.random.default_rng(np.random.PCG64([seed, 0x5151]))
    parent = [-1]
    length = [root_len]
    start = [0]
    children: List[List[int]] = [[]]
    leaves = 1
    while leaves < n_leaves:
        lens = np.asarray(length, dtype=np.float64)
        splittable = lens >= 2
        while True:
            p = (lens * splittable) / (lens * splittable).sum()
            j = int(rng.choice(len(length), p=p))
            o = int(rng.integers(1, length[j]))
            if (start[j] + o) % chunk != 0:
                break
        # split j at offset o: j keeps [0, o), new segment b gets [o, len) and j's children
        b = len(parent)
        parent.append(j)
        length.append(length[j] - o)
        start.append(start[j] + o)
        children.append(children[j])
        for c in children[j]:
            parent[c] = b
        children[j] = [b]
        length[j] = o
        f = int(rng.integers(2, 5))
        f = min(f, n_leaves - leaves + 1)
        for _ in range(f - 1):
            ln = int(round(float(np.exp(rng.uniform(np.log(min_leaf), np.log(max_leaf))))))
            c = len(parent)
            parent.append(j)
            length.append(ln)
            start.append(start[j] + o)
            children.append([])
            children[j].append(c)
        leaves += f - 1
    return GenTree(parent=parent, length=length).finalize(seed=seed)


def random_small_tree(rng: np.random.Generator, max_segments: int = 8, max_len: int = 40,
                      forest: bool = False) -> GenTree:
    """A random tree of at most ``max_segments`` segments for brute-force checks.

    Every internal segment gets at least two children (a segment with one
    child would not be fork-free-maximal).  Lengths are uniform in
    [1, max_len]; with ``forest`` the roots may be several.
    """
    n_target = int(rng.integers(1, max_segments + 1))
    parent = [-1]
    if forest and n_target >= 2 and rng.random() < 0.3:
        parent = [-1, -1]
    while len(parent) < n_target:
        leaves = [j for j in range(len(parent)) if j not in parent]
        internal = [j for j in range(len(parent)) if j in parent]
        room = n_target - len(parent)
        if internal and rng.random() < 0.3:
            p = int(rng.choice(internal))
            parent.append(p)
        elif room >= 2:
            p = int(rng.choice(leaves))
            k = int(rng.integers(2, min(4, room) + 1))
            parent.extend([p] * k)
        else:
            if internal:
                parent.append(int(rng.choice(internal)))
            else:
                break
    length = [int(rng.integers(1, max_len + 1)) for _ in parent]
    return GenTree(parent=parent, length=length).finalize(seed=int(rng.integers(0, 2**31)))


def forest_of_sequences(lengths: Sequence[int], seed: int = 0) -> GenTree:
    """Independent sequences (one root segment each), e.g. a flat packed batch."""
    return GenTree(parent=[-1] * len(lengths), length=list(lengths)).finalize(seed=seed, shuffle=False)


def flat_varlen_lengths(seed: int = 0, n: int = 32, lo: int = 1024, hi: int = 4096, chunk: int = 64) -> np.ndarray:
    """Lengths of the flat packed batch: uniform in [lo, hi], multiples of
    ``chunk`` rejected."""
    rng = np.random.default_rng(np.random.PCG64([seed, 0x1111]))
    out = []
    while len(out) < n:
        L = int(rng.integers(lo, hi + 1))
        if L % chunk:
            out.append(L)
    return np.asarray(out, dtype=np.int64)
