"""Pins of the oracle planner against things other than itself: brute force,
closed forms, direct prefix comparison and the pages' figure examples."""
import json
import os

import numpy as np
import pytest

from oracle import planner
from synthetic import trees

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lcp(a, b):
    n = min(len(a), len(b))
    i = 0
    while i < n and a[i] == b[i]:
        i += 1
    return i


def _compact_by_lcp(t):
    """C = sum |x| - sum of LCPs of lexicographically adjacent trajectories
    (paperlayer summary, section 3: splitting between sorted neighbours costs
    their LCP; compact work = unique token nodes)."""
    trajs = [tuple(t.trajectory(i).tolist()) for i in range(t.n_traj)]
    trajs.sort()
    return sum(len(x) for x in trajs) - sum(_lcp(trajs[i], trajs[i + 1]) for i in range(len(trajs) - 1))


def _gen_trees():
    out = [trees.tiny_tree("G"), trees.tiny_tree("D"), trees.figure1_tree(), trees.figure2_tree(),
           trees.figureC1_tree()]
    rng = np.random.default_rng(5)
    for _ in range(30):
        out.append(trees.random_small_tree(rng, max_segments=8, max_len=40, forest=True))
    # degenerate: duplicates and a trajectory that is a prefix of another
    g = trees.GenTree(parent=[-1, 0, 0], length=[30, 10, 12], extra_ends=[(0, 17), (1, 4)], duplicates=[0])
    out.append(g.finalize(seed=3))
    out.append(trees.GenTree(parent=[-1], length=[1]).finalize())
    return out


@pytest.mark.parametrize("idx", range(37))
def test_compact_count_equals_lcp_formula_and_generator(idx):
    t = _gen_trees()[idx]
    p = planner.make_plan(t.tokens, t.offsets, 16)
    assert p.C == _compact_by_lcp(t)
    # the generator's own node count (siblings have distinct first tokens)
    assert p.C == len(np.unique(t.node_of_pos))
    # the partition of semantic positions by m equals the generator's node partition
    pairs = set(zip(p.m.tolist(), t.node_of_pos.tolist()))
    assert len(pairs) == p.C
    assert p.q.sum() == p.S == t.S
    assert np.array_equal(p.q, np.bincount(p.m, minlength=p.C))
    assert (p.q >= 1).all()


def test_c2_ratio_matches_generator_counts():
    t = trees.random_rollout_tree(seed=0)
    p = planner.make_plan(t.tokens, t.offsets, 64)
    assert p.C == t.n_nodes == sum(t.length)
    assert p.S == int(t.offsets[-1])
    lens = np.diff(t.offsets)
    assert len(lens) == 64
    assert p.min_calls == p.n_rounds
    assert len(p.seqs) == 64
    assert p.replay_total == planner.forced_replay_total(p.segments, 64)
    # every side branch replays fewer than B tokens
    assert all(len(s.replay_rows) < 64 for s in p.seqs)


@pytest.mark.parametrize("B", [4, 8, 16])
def test_min_calls_equals_brute_force(B):
    rng = np.random.default_rng(100 + B)
    n = 0
    for _ in range(700):
        t = trees.random_small_tree(rng, max_segments=8, max_len=3 * B, forest=True)
        trie = planner.build_trie(t.tokens, t.offsets)
        seg = planner.build_segments(trie)
        assert len(seg.nodes) <= 8
        mc = planner.min_calls(seg, B)
        assert mc == planner.brute_force_min_calls(seg, B)
        n += 1
    assert n == 700


@pytest.mark.parametrize("B", [4, 16])
def test_recovered_plan_is_minimal_and_well_formed(B):
    rng = np.random.default_rng(7 + B)
    for _ in range(200):
        t = trees.random_small_tree(rng, max_segments=8, max_len=3 * B, forest=True)
        p = planner.make_plan(t.tokens, t.offsets, B)
        seg = p.segments
        assert p.n_rounds == p.min_calls
        leaves = sum(1 for v in range(len(seg.nodes)) if not seg.children[v])
        assert len(p.seqs) == leaves
        assert p.replay_total == planner.forced_replay_total(seg, B)
        rows = np.concatenate([s.own_rows for s in p.seqs])
        assert np.array_equal(rows, np.arange(p.C))
        for i, s in enumerate(p.seqs):
            assert s.start % B == 0
            assert len(s.replay_rows) == seg.start[s.head] - s.start < B
            if s.init_slot >= 0:
                prod = p.slot_producer[s.init_slot]
                assert p.seqs[prod].round < s.round
                assert (s.start - p.seqs[prod].start) // B in dict(p.seqs[prod].emits)
            else:
                assert s.start == 0


def _named_plan(spec):
    names = list(spec["segments"].keys())
    parent = [(-1 if spec["segments"][n][0] is None else names.index(spec["segments"][n][0])) for n in names]
    length = [spec["segments"][n][1] for n in names]
    t = trees.GenTree(parent=parent, length=length).finalize(seed=11)
    p = planner.make_plan(t.tokens, t.offsets, spec["B"])
    # map oracle segments to names through their first node's generator id
    first_node = {}
    for v in range(len(p.segments.nodes)):
        nd = p.segments.nodes[v][0]
        s = int(np.nonzero(p.trie.m_node == nd)[0][0])
        gen = int(t.node_of_pos[s])
        j = int(np.searchsorted(t.node_base, gen, side="right") - 1)
        first_node[v] = names[j]
    return t, p, first_node


@pytest.mark.parametrize("fig", ["figure1", "figure2", "figureC1"])
def test_figure_call_assignments(fig):
    spec = json.load(open(os.path.join(GOLDEN, "figure_calls.json")))[fig]
    t, p, name = _named_plan(spec)
    got = []
    for r in range(1, p.n_rounds + 1):
        got.append(sorted([[name[v] for v in p.seqs[i].segs] for i in p.round_seqs(r)]))
    want = [sorted(c) for c in spec["calls"]]
    assert got == want
    for seg_name, rep in spec.get("replay", {}).items():
        s = [s for s in p.seqs if name[s.head] == seg_name][0]
        assert len(s.replay_rows) == rep
    if "shared_initial_state" in spec:
        slots = {s.init_slot for s in p.seqs if name[s.head] in spec["shared_initial_state"]}
        assert len(slots) == 1 and -1 not in slots
    for seg_name, mult in spec.get("multiplicity", {}).items():
        v = [v for v in name if name[v] == seg_name][0]
        rows = p.m[np.isin(p.trie.m_node, p.segments.nodes[v])]
        assert set(p.q[rows].tolist()) == {mult}


def test_forced_replay_independent_of_continuation_choice():
    rng = np.random.default_rng(3)
    B = 8
    for _ in range(100):
        t = trees.random_small_tree(rng, max_segments=8, max_len=30)
        trie = planner.build_trie(t.tokens, t.offsets)
        seg = planner.build_segments(trie)
        forks = [v for v in range(len(seg.nodes)) if seg.children[v]]
        R = planner.forced_replay_total(seg, B)
        for _k in range(5):
            cont = {v: seg.children[v][int(rng.integers(len(seg.children[v])))] for v in forks}
            tot = 0
            for v in forks:
                for c in seg.children[v]:
                    if cont[v] != c:
                        tot += seg.start[c] - planner.anchor(seg.start[c], B)
            assert tot == R


def test_chunk_aligned_forks_replay_nothing():
    # fork exactly at a multiple of B: side branches replay 0 tokens
    t = trees.GenTree(parent=[-1, 0, 0, 0], length=[64, 10, 20, 30]).finalize(seed=1)
    p = planner.make_plan(t.tokens, t.offsets, 64)
    assert p.replay_total == 0
    assert p.n_rounds == 2
    side = [s for s in p.seqs if s.round == 2]
    assert len(side) == 2 and all(len(s.replay_rows) == 0 for s in side)
    assert len({s.init_slot for s in side}) == 1


def test_fork_before_first_boundary_starts_in_round_one():
    # fork at p < B on a pre-ready root that crosses no boundary: one call
    t = trees.GenTree(parent=[-1, 0, 0, 0], length=[20, 10, 20, 30]).finalize(seed=2)
    p = planner.make_plan(t.tokens, t.offsets, 64)
    assert p.n_rounds == 1
    assert p.n_slots == 0
    assert sorted(len(s.replay_rows) for s in p.seqs) == [0, 20, 20]
