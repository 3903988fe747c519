"""Oracle planner -- test infrastructure (see ``oracle/__init__.py``).

Written from the HARTS pages (arXiv 2608.28158):

* compact tokens and the map m: S -> C -- the close-reading blog, section 3.2
  (semantic positions s=(x,i), compact tokens, the dedup coordinate system);
  paperlayer summary, section 3 (compact trie work = number of unique token
  nodes);
* multiplicity q_c = number of semantic positions on compact token c, summing
  to S -- blog section 4.4;
* fork-free segments, the packed chunkwise call model (at most one direct
  continuation per fork; a state produced inside a call initialises another
  sequence only after the call returns), T_pre / T_in with leaves = 1 and the
  minimum call count T_pre(root), top-down recovery, replay of [a(p), p) --
  blog section 4.2; Figure 2 of the thelatestinai page (three boundary cases);
* compact physical layout (sequence tokens contiguous, one packed call per
  round, replay sources and requested states addressable) -- blog section 4.3.

The pages cite but do not print equations (13)-(14).  The recursion below is
the plainest reading consistent with "direct continuation does not wait, side
branches are delayed one round" and the three boundary cases:

    X(v)     = a chunk boundary lies in (s_v, e_v]
    F(v)     = min_d max(T_in(d), 1 + max_{c != d} T_pre(c))
    T_in(v)  = F(v)
    T_pre(v) = max_c T_pre(c) if not X(v) else F(v)
    leaves: T_pre = T_in = 1

It is checked against :func:`brute_force_min_calls`, an exhaustive search
over every continuation choice under the execution model itself.

Canonical choices (needed for bit-exact plans, where the pages are silent):
children ordered by first token id; the direct continuation is the first child
minimising F (or simply the first child when v's entry anchor is ready and v
crosses no boundary); every sequence runs in its earliest legal round;
sequences in a round are ordered by the DFS preorder of their head segment;
compact rows are round-major, then sequence, then path order; slots are
numbered in first-use order (round, then sequence) and keyed by the compact row
of the token just before the anchor.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np


# ----------------------------------------------------------------------------- trie

@dataclass
class Trie:
    parent: List[int]          # trie node -> parent node (-1 for the empty root's children)
    token: List[int]           # token id of the node
    depth: List[int]           # absolute position of the node (0-based)
    children: List[List[int]]  # ordered by token id
    roots: List[int]           # children of the empty prefix, ordered by token id
    m_node: np.ndarray         # semantic position -> trie node
    S: int

    @property
    def C(self) -> int:
        return len(self.parent)


def build_trie(tokens: np.ndarray, offsets: np.ndarray) -> Trie:
    """Distinct prefixes of the trajectories: node(x, i) = child(node(x, i-1), x[i]).

    This is the plain definition of the compact token set (each distinct prefix
    is one compact token)."""
    key_to_node: Dict[Tuple[int, int], int] = {}
    parent: List[int] = []
    token: List[int] = []
    depth: List[int] = []
    S = int(offsets[-1])
    m_node = np.empty(S, dtype=np.int64)
    for x in range(len(offsets) - 1):
        prev = -1
        for s in range(int(offsets[x]), int(offsets[x + 1])):
            key = (prev, int(tokens[s]))
            node = key_to_node.get(key)
            if node is None:
                node = len(parent)
                key_to_node[key] = node
                parent.append(prev)
                token.append(int(tokens[s]))
                depth.append(0 if prev < 0 else depth[prev] + 1)
            m_node[s] = node
            prev = node
    children: List[List[int]] = [[] for _ in parent]
    roots: List[int] = []
    for n, p in enumerate(parent):
        (roots if p < 0 else children[p]).append(n)
    for lst in children:
        lst.sort(key=lambda n: token[n])
    roots.sort(key=lambda n: token[n])
    return Trie(parent, token, depth, children, roots, m_node, S)


def trie_dfs_preorder(trie: Trie) -> List[int]:
    out: List[int] = []
    stack = list(reversed(trie.roots))
    while stack:
        n = stack.pop()
        out.append(n)
        stack.extend(reversed(trie.children[n]))
    return out


# ------------------------------------------------------------------------- segments

@dataclass
class Segments:
    nodes: List[List[int]]      # trie nodes of each segment, in path order
    start: List[int]            # s_v
    end: List[int]              # e_v
    children: List[List[int]]   # child segments, ordered by first token id
    parent: List[int]
    roots: List[int]            # root segments, ordered by first token id
    preorder: List[int]         # segment DFS preorder
    pre_id: List[int]           # segment -> position in preorder


def build_segments(trie: Trie) -> Segments:
    """Maximal fork-free token paths: a node continues its parent's segment iff
    the parent has exactly one child."""
    seg_of = [-1] * trie.C
    nodes: List[List[int]] = []
    start: List[int] = []
    parent: List[int] = []
    heads = list(trie.roots)
    head_parent = [-1] * len(heads)
    children_by_seg: List[List[int]] = []
    i = 0
    while i < len(heads):
        h = heads[i]
        sid = len(nodes)
        path = [h]
        n = h
        while len(trie.children[n]) == 1:
            n = trie.children[n][0]
            path.append(n)
        for x in path:
            seg_of[x] = sid
        nodes.append(path)
        start.append(trie.depth[h])
        parent.append(head_parent[i])
        children_by_seg.append([])
        if head_parent[i] >= 0:
            children_by_seg[head_parent[i]].append(sid)
        for c in trie.children[n]:  # >= 2 children (fork) or none (leaf)
            heads.append(c)
            head_parent.append(sid)
        i += 1
    end = [start[v] + len(nodes[v]) for v in range(len(nodes))]
    first_tok = [trie.token[nodes[v][0]] for v in range(len(nodes))]
    for lst in children_by_seg:
        lst.sort(key=lambda v: first_tok[v])
    roots = sorted([v for v in range(len(nodes)) if parent[v] < 0], key=lambda v: first_tok[v])
    preorder: List[int] = []
    stack = list(reversed(roots))
    while stack:
        v = stack.pop()
        preorder.append(v)
        stack.extend(reversed(children_by_seg[v]))
    pre_id = [0] * len(nodes)
    for i, v in enumerate(preorder):
        pre_id[v] = i
    return Segments(nodes, start, end, children_by_seg, parent, roots, preorder, pre_id)


def anchor(p: int, B: int) -> int:
    """a(p): the chunk boundary at or before absolute position p."""
    return B * (p // B)


def crosses(seg: Segments, v: int, B: int) -> bool:
    """X(v): a chunk boundary lies in (s_v, e_v]."""
    return seg.end[v] // B > seg.start[v] // B


# ------------------------------------------------------------------- T_pre / T_in

def min_calls_tables(seg: Segments, B: int) -> Tuple[List[int], List[int], List[int]]:
    """Bottom-up T_pre, T_in and F for every segment (leaves: 1, 1, 1)."""
    n = len(seg.nodes)
    T_pre = [0] * n
    T_in = [0] * n
    F = [0] * n
    for v in reversed(seg.preorder):  # children before parents
        ch = seg.children[v]
        if not ch:
            T_pre[v] = T_in[v] = F[v] = 1
            continue
        best = None
        for d in ch:
            others = [T_pre[c] for c in ch if c != d]
            val = max(T_in[d], 1 + max(others)) if others else T_in[d]
            if best is None or val < best:
                best = val
        F[v] = best
        T_in[v] = F[v]
        T_pre[v] = max(T_pre[c] for c in ch) if not crosses(seg, v, B) else F[v]
    return T_pre, T_in, F


def min_calls(seg: Segments, B: int) -> int:
    T_pre, _, _ = min_calls_tables(seg, B)
    return max(T_pre[r] for r in seg.roots)


# --------------------------------------------------------------- execution model

def _path_rows_before(seg: Segments, v: int, lo: int, hi: int) -> List[Tuple[int, int]]:
    """(segment, offset) of the absolute positions [lo, hi) on the path to v."""
    out: List[Tuple[int, int]] = []
    u = v
    while u >= 0:
        for p in range(max(lo, seg.start[u]), min(hi, seg.end[u])):
            out.append((u, p - seg.start[u]))
        u = seg.parent[u]
    out.sort(key=lambda t: seg.start[t[0]] + t[1])
    return out


def simulate_rounds(seg: Segments, cont: Dict[int, Optional[int]], B: int) -> Dict[int, int]:
    """Earliest legal round of every sequence head under the packed chunkwise
    call model, for a given choice of direct continuation per fork.

    A sequence headed by segment h starts from the state at a = a(s_h): the zero
    state when a = 0, otherwise the state emitted by the sequence that owns the
    token at position a-1 on h's path, usable only after that sequence's call
    returns."""
    head_of: Dict[int, int] = {}
    heads: List[int] = []
    for v in seg.preorder:
        p = seg.parent[v]
        if p >= 0 and cont.get(p) == v:
            head_of[v] = head_of[p]
        else:
            head_of[v] = v
            heads.append(v)
    rounds: Dict[int, int] = {}

    def rnd(h: int) -> int:
        if h in rounds:
            return rounds[h]
        a = anchor(seg.start[h], B)
        if a == 0:
            r = 1
        else:
            # owner of position a-1 on h's path
            u = seg.parent[h]
            while not (seg.start[u] <= a - 1 < seg.end[u]):
                u = seg.parent[u]
            r = rnd(head_of[u]) + 1
        rounds[h] = r
        return r

    for h in heads:
        rnd(h)
    return rounds


def brute_force_min_calls(seg: Segments, B: int) -> int:
    """Minimum number of rounds over every choice of direct continuation
    (including none) at every fork."""
    forks = [v for v in range(len(seg.nodes)) if seg.children[v]]
    options = [[None] + list(seg.children[v]) for v in forks]
    best = None
    for choice in itertools.product(*options):
        cont = dict(zip(forks, choice))
        r = max(simulate_rounds(seg, cont, B).values())
        if best is None or r < best:
            best = r
    return best


# ------------------------------------------------------------------------ the plan

@dataclass
class SeqPlan:
    head: int                 # head segment
    segs: List[int]           # continuation chain, head first
    round: int                # 1-based
    start: int                # absolute anchor a(s_head): start of the virtual stream
    own_rows: List[int] = field(default_factory=list)     # compact rows, path order
    replay_rows: List[int] = field(default_factory=list)  # compact rows of [start, s_head)
    init_slot: int = -1
    emits: List[Tuple[int, int]] = field(default_factory=list)  # (boundary index, slot)


@dataclass
class Plan:
    B: int
    S: int
    C: int
    n_rounds: int
    seqs: List[SeqPlan]              # ordered: round-major, then head DFS preorder
    m: np.ndarray                    # int64 [S] semantic position -> compact row
    q: np.ndarray                    # int32 [C]
    node_to_row: np.ndarray          # int64 [C] trie-node DFS preorder index -> compact row
    row_pos: np.ndarray              # int64 [C] absolute position of each compact row
    n_slots: int
    slot_row: List[int]              # compact row of the token before each slot's anchor
    slot_producer: List[int]         # sequence index producing each slot
    min_calls: int
    replay_total: int
    trie: Trie
    segments: Segments

    def round_seqs(self, r: int) -> List[int]:
        return [i for i, s in enumerate(self.seqs) if s.round == r]


def make_plan(tokens: np.ndarray, offsets: np.ndarray, B: int) -> Plan:
    trie = build_trie(tokens, offsets)
    seg = build_segments(trie)
    T_pre, T_in, F = min_calls_tables(seg, B)
    # top-down recovery of continuation choices with entry-anchor readiness
    cont: Dict[int, Optional[int]] = {}
    ready = {r: True for r in seg.roots}
    for v in seg.preorder:
        ch = seg.children[v]
        if not ch:
            continue
        if ready[v] and not crosses(seg, v, B):
            d = ch[0]
            d_ready = True
        else:
            best, d = None, None
            for c in ch:
                others = [T_pre[x] for x in ch if x != c]
                val = max(T_in[c], 1 + max(others)) if others else T_in[c]
                if best is None or val < best:
                    best, d = val, c
            d_ready = False
        cont[v] = d
        for c in ch:
            ready[c] = d_ready if c == d else True
    rounds = simulate_rounds(seg, cont, B)
    n_rounds = max(rounds.values())
    mc = max(T_pre[r] for r in seg.roots)
    # sequences
    seqs: List[SeqPlan] = []
    for h in sorted(rounds, key=lambda h: (rounds[h], seg.pre_id[h])):
        chain = [h]
        while chain[-1] in cont:
            chain.append(cont[chain[-1]])
        seqs.append(SeqPlan(head=h, segs=chain, round=rounds[h], start=anchor(seg.start[h], B)))
    # compact rows: round-major, sequence order, path order
    node_row = np.full(trie.C, -1, dtype=np.int64)
    row_pos = np.zeros(trie.C, dtype=np.int64)
    row = 0
    for sp in seqs:
        for v in sp.segs:
            for nd in seg.nodes[v]:
                node_row[nd] = row
                row_pos[row] = trie.depth[nd]
                sp.own_rows.append(row)
                row += 1
    assert row == trie.C
    # replay rows
    for sp in seqs:
        if seg.start[sp.head] > sp.start:
            for (u, off) in _path_rows_before(seg, sp.head, sp.start, seg.start[sp.head]):
                sp.replay_rows.append(int(node_row[seg.nodes[u][off]]))
    # slots, first-use order
    row_owner = np.empty(trie.C, dtype=np.int64)
    for i, sp in enumerate(seqs):
        row_owner[sp.own_rows] = i
    slot_of_row: Dict[int, int] = {}
    slot_row: List[int] = []
    slot_producer: List[int] = []
    for i, sp in enumerate(seqs):
        a = sp.start
        if a == 0:
            continue
        (u, off) = _path_rows_before(seg, sp.head, a - 1, a)[0]
        key = int(node_row[seg.nodes[u][off]])
        if key not in slot_of_row:
            slot_of_row[key] = len(slot_row)
            slot_row.append(key)
            prod = int(row_owner[key])
            slot_producer.append(prod)
            b = (a - seqs[prod].start)
            assert b % B == 0 and b > 0
            seqs[prod].emits.append((b // B, slot_of_row[key]))
        sp.init_slot = slot_of_row[key]
    for sp in seqs:
        sp.emits.sort()
    m = node_row[trie.m_node]
    q = np.bincount(m, minlength=trie.C).astype(np.int32)
    pre = trie_dfs_preorder(trie)
    node_to_row = node_row[np.asarray(pre, dtype=np.int64)]
    replay_total = sum(len(sp.replay_rows) for sp in seqs)
    return Plan(B=B, S=trie.S, C=trie.C, n_rounds=n_rounds, seqs=seqs, m=m, q=q,
                node_to_row=node_to_row, row_pos=row_pos, n_slots=len(slot_row), slot_row=slot_row,
                slot_producer=slot_producer, min_calls=mc, replay_total=replay_total, trie=trie,
                segments=seg)


def forced_replay_total(seg: Segments, B: int) -> int:
    """R = sum over forks v of (|ch(v)| - 1) * (e_v mod B): the replay length is
    fixed by the fork position and does not depend on the continuation choice
    (blog section 4.2)."""
    return sum((len(seg.children[v]) - 1) * (seg.end[v] % B)
               for v in range(len(seg.nodes)) if seg.children[v])
