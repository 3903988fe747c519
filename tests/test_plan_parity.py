"""Bit-exact parity of the C-ABI planner (host C++) with the oracle planner:
maps m and q, trie-node -> row, rounds, sequences, replay rows, slots and
emitted-state requests, on figure trees, random trees, degenerate inputs and
the 64-leaf rollout workload."""
import numpy as np
import pytest

import chunkwise_linear_attention_gated_amd as harts
from oracle import planner
from synthetic import trees


def _compare(t, B):
    op = planner.make_plan(t.tokens, t.offsets, B)
    hp = harts.TreePlan(t.tokens, t.offsets, B)
    inf = hp.info
    assert (inf.S, inf.C, inf.n_rounds, inf.min_calls) == (op.S, op.C, op.n_rounds, op.min_calls)
    assert (inf.n_sequences, inf.n_slots, inf.replay_total) == (len(op.seqs), op.n_slots, op.replay_total)
    m, q, n2r = hp.maps()
    assert np.array_equal(m, op.m)
    assert np.array_equal(q, op.q)
    assert np.array_equal(n2r, op.node_to_row)
    seqs = hp.sequences()
    rep = hp.replay_rows()
    eb, et = hp.emits()
    for s, o in zip(seqs, op.seqs):
        assert s["round"] == o.round and s["start"] == o.start and s["init_slot"] == o.init_slot
        assert (s["row_begin"], s["row_end"]) == (o.own_rows[0], o.own_rows[-1] + 1)
        assert list(rep[s["replay_off"]:s["replay_off"] + s["n_replay"]]) == o.replay_rows
        em = list(zip(eb[s["emit_off"]:s["emit_off"] + s["n_emits"]].tolist(),
                      et[s["emit_off"]:s["emit_off"] + s["n_emits"]].tolist()))
        assert em == o.emits
    _compare_rounds(hp, op)
    st = hp.tree_stats()
    assert st["n_segments"] == len(op.segments.nodes)
    return op


def _compare_rounds(hp, op):
    """harts_plan_round: round r's sequences, in plan order, with their replay rows and emits."""
    for r in range(op.n_rounds):
        rv = hp.round(r)
        mine = [o for o in op.seqs if o.round == r + 1]
        assert rv["n_seq"] == len(mine)
        for i, o in enumerate(mine):
            assert (rv["row_start"][i], rv["row_end"][i]) == (o.own_rows[0], o.own_rows[-1] + 1)
            assert rv["abs_start"][i] == o.start and rv["init_slot"][i] == o.init_slot
            a, b = rv["replay_off"][i:i + 2]
            assert list(rv["replay_rows"][a:b]) == o.replay_rows
            a, b = rv["emit_off"][i:i + 2]
            assert list(zip(rv["emit_chunk"][a:b].tolist(), rv["emit_slot"][a:b].tolist())) == o.emits
    for bad in (-1, op.n_rounds):
        with pytest.raises(harts.HartsError) as e:
            hp.round(bad)
        assert e.value.code == -1 and "outside" in str(e.value)


@pytest.mark.parametrize("B", [16, 32, 64])
def test_fixed_trees(B):
    for t in [trees.tiny_tree("G"), trees.tiny_tree("D"), trees.figure1_tree(), trees.figure2_tree(),
              trees.figureC1_tree()]:
        _compare(t, B)


@pytest.mark.parametrize("B", [16, 32, 64])
def test_random_trees(B):
    rng = np.random.default_rng(1000 + B)
    for _ in range(300):
        t = trees.random_small_tree(rng, max_segments=10, max_len=3 * B, forest=True)
        _compare(t, B)


def test_degenerate_inputs():
    # single trajectory; duplicates; a trajectory that is a prefix of another;
    # forks exactly on chunk boundaries; forks before the first boundary
    cases = [
        trees.GenTree(parent=[-1], length=[1]).finalize(),
        trees.GenTree(parent=[-1], length=[200]).finalize(),
        trees.GenTree(parent=[-1, 0, 0], length=[30, 10, 12], extra_ends=[(0, 17), (1, 4)], duplicates=[0, 1]).finalize(seed=4),
        trees.GenTree(parent=[-1, 0, 0, 0], length=[64, 10, 20, 30]).finalize(seed=1),
        trees.GenTree(parent=[-1, 0, 0, 1, 1], length=[128, 64, 3, 64, 1]).finalize(seed=5),
        trees.GenTree(parent=[-1, 0, 0, 0], length=[20, 10, 20, 30]).finalize(seed=2),
        trees.GenTree(parent=[-1, -1, -1], length=[5, 70, 64]).finalize(seed=6),
    ]
    for t in cases:
        for B in (16, 64):
            _compare(t, B)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rollout_workload(seed):
    t = trees.random_rollout_tree(seed=seed)
    op = _compare(t, 64)
    assert len(op.seqs) == 64
    assert all(len(s.replay_rows) < 64 for s in op.seqs)


def test_varlen_plan():
    lens = trees.flat_varlen_lengths(seed=0, n=32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    has = (np.arange(32) % 2 == 1).astype(np.uint8)
    vp = harts.VarlenPlan(cu, 64, has_init=has, emit_boundaries=True)
    inf = vp.info
    assert inf.n_rounds == 1 and inf.n_sequences == 32 and inf.C == cu[-1]
    bo = vp.boundary_offsets()
    assert np.array_equal(np.diff(bo), lens // 64)
    assert inf.n_boundaries == int((lens // 64).sum())
    seqs = vp.sequences()
    assert [s["init_slot"] for s in seqs] == [i if has[i] else -1 for i in range(32)]
    m, q, n2r = vp.maps()
    assert np.array_equal(m, np.arange(cu[-1])) and (q == 1).all()
    rv = vp.round(0)
    assert rv["n_seq"] == 32 and np.array_equal(rv["row_start"], cu[:-1]) and np.array_equal(rv["row_end"], cu[1:])
    assert np.array_equal(rv["abs_start"], np.zeros(32)) and len(rv["replay_rows"]) == 0
    assert np.array_equal(np.diff(rv["emit_off"]), lens // 64)
