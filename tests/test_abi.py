"""The C ABI library loads, exports every symbol include/harts.h declares, and
turns bad host-side inputs into error codes (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import chunkwise_linear_attention_gated_amd as harts
from chunkwise_linear_attention_gated_amd import _lib
from synthetic import trees

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "harts.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(harts_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(_lib.library)
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n


def test_version():
    assert "gfx950" in harts.version()


def test_error_codes():
    with pytest.raises(harts.HartsError) as e:
        harts.TreePlan(np.array([1, 2, 3], np.int32), np.array([0, 3, 3], np.int64), 64)
    assert e.value.code == -1 and "empty trajectory" in str(e.value)
    with pytest.raises(harts.HartsError) as e:
        harts.TreePlan(np.array([1, 2, 3], np.int32), np.array([0, 3], np.int64), 48)
    assert e.value.code == -1 and "chunk_B" in str(e.value)
    with pytest.raises(harts.HartsError):
        harts.VarlenPlan(np.array([0, 5, 4], np.int64), 64)
    with pytest.raises(harts.HartsError):
        harts.VarlenPlan(np.array([1, 5], np.int64), 64)


def test_unsupported_shapes_rejected_before_any_device_work():
    p = harts.TreePlan(np.array([1, 2, 3], np.int32), np.array([0, 3], np.int64), 64)
    with pytest.raises(harts.HartsError) as e:
        harts.DevicePlan(p, 2, 48, 48, harts.DTYPE_BF16, stream=0)
    assert "unsupported" in str(e.value)
    with pytest.raises(harts.HartsError):
        harts.DevicePlan(p, 0, 128, 128, harts.DTYPE_BF16, stream=0)


def test_logprob_rows_is_the_stable_inverse_of_m():
    from oracle import logprob as olp
    rng = np.random.default_rng(3)
    for C, S in [(1, 0), (5, 1), (9, 60), (40, 300)]:
        m = rng.integers(0, C, size=S)
        off, pos = harts.logprob_rows(m, C)
        want_off, want_pos = olp.rows_of_map(m, C)
        assert np.array_equal(off, want_off) and np.array_equal(pos, want_pos)
    with pytest.raises(harts.HartsError) as e:
        harts.logprob_rows(np.array([0, 3, 1]), 3)
    assert e.value.code == -1 and "outside" in str(e.value)


def test_logprob_workspace_takes_compact_and_semantic_sizes():
    for C, S in [(0, 0), (1, 5), (4097, 100000)]:
        assert harts.logprob_workspace(C, S) == harts.logprob_workspace_size(C)
    assert harts.logprob_workspace(4097, 1) % 256 == 0 and harts.logprob_workspace(4097, 1) >= 4097 * 4


def test_kda_fwd_varlen_rejects_bad_arguments_before_any_device_work():
    f = _lib._kda_fwd_varlen
    assert f(None, None) == -1
    a = _lib.VarlenArgs()
    assert f(ctypes.byref(a), None) == -1 and b"cu_seqlens" in _lib._last_error()
    cu = np.array([0, 5, 3], np.int64)
    a.cu_seqlens, a.n_seq, a.H, a.dk, a.dv, a.chunk_B = cu.ctypes.data, 2, 2, 128, 128, 64
    assert f(ctypes.byref(a), None) == -1 and b"required" in _lib._last_error()  # no tensors
    # stand-in addresses: every case below is refused on the host, before any of them is used
    a.q = a.k = a.v = a.g = a.beta = a.o = 256
    assert f(ctypes.byref(a), None) == -1 and b"decreasing" in _lib._last_error()  # the plan is refused
    cu2 = np.array([0, 5, 9], np.int64)
    a.cu_seqlens, a.dk, a.dv = cu2.ctypes.data, 48, 48
    assert f(ctypes.byref(a), None) == -1 and b"unsupported" in _lib._last_error()


def test_logprob_map_check_names_the_first_position_out_of_range():
    m = np.array([0, 2, 1, 2], np.int64)
    lab = np.array([5, 0, 9, 3], np.int32)
    harts.logprob_check_map(m, lab, 3, 10)
    harts.logprob_check_map(m, None, 3, 1)
    with pytest.raises(harts.HartsError) as e:
        harts.logprob_check_map(np.array([0, 3, -1], np.int64), None, 3, 10)
    assert e.value.code == -2 and "m[1]" in str(e.value)
    with pytest.raises(harts.HartsError) as e:
        harts.logprob_check_map(m, np.array([5, 0, 10, -1], np.int32), 3, 10)
    assert e.value.code == -2 and "labels[2]" in str(e.value)
    with pytest.raises(harts.HartsError) as e:
        harts.logprob_check_map(m, np.array([5, -1, 0, 0], np.int32), 3, 10)
    assert "labels[1]" in str(e.value)


def test_logprob_backward_rejects_bad_arguments_before_any_device_work():
    f = _lib._lpb
    assert f(None, 4, 0, 0, None, None, None, None, None, 0, None, None) == -1  # V < 1
    assert f(None, 4, 8, 7, None, None, None, None, None, 0, None, None) == -1  # unknown dtype
    assert f(None, 4, 8, 0, None, None, None, None, None, 0, None, None) == -1  # missing arrays
    assert b"required" in _lib._last_error()
    assert f(None, 0, 8, 0, None, None, None, None, None, 0, None, None) == 0  # no rows: nothing to do


def test_conv_tables_follow_each_trajectory():
    # trajectories [a b c d e] [a b c f] [a b g h]: rows a..h = 0..7
    m = np.array([0, 1, 2, 3, 4, 0, 1, 2, 5, 0, 1, 6, 7])
    off = np.array([0, 5, 9, 13])
    anc, goff, gl = harts.conv_tables(m, off, 8, 3)
    want = np.array([[-1, -1], [0, -1], [1, 0], [2, 1], [3, 2], [2, 1], [1, 0], [6, 1]])
    assert np.array_equal(anc, want)
    # gather lists: the (t, j) with anc_j(t) = s, increasing (j, t)
    got = {s: [(int(e) >> 3, int(e) & 7) for e in gl[goff[s]:goff[s + 1]]] for s in range(8)}
    assert got[1] == [(2, 1), (6, 1), (3, 2), (5, 2), (7, 2)]
    assert got[0] == [(1, 1), (2, 2), (6, 2)] and got[4] == [] and got[7] == []
    with pytest.raises(harts.HartsError) as e:  # row 2 preceded by 1 on one trajectory and by 0 on another
        harts.conv_tables(np.array([0, 1, 2, 0, 2]), np.array([0, 3, 5]), 3, 2)
    assert "prefix tree" in str(e.value)
    with pytest.raises(harts.HartsError) as e:
        harts.conv_tables(np.array([0, 1]), np.array([0, 2]), 3, 2)
    assert "no trajectory" in str(e.value)
    with pytest.raises(harts.HartsError):
        harts.conv_tables(m, off, 8, 9)


def _attn_check_tables(m, off, C):
    from oracle import attention as oatt
    tb = harts.attn_tables(m, off, C)
    P = oatt.paths(m, off, C)
    qt, kv, kt, ql = tb["qtiles"], tb["kv_list"], tb["ktiles"], tb["q_list"]
    seen_q = np.zeros(C, np.int64)
    for row0, n, o, base in qt:
        assert 1 <= n <= 128
        for i in range(n):
            seen_q[row0 + i] += 1
            assert list(kv[o:o + base + i + 1]) == list(P[row0 + i])  # the path, root first
    assert (seen_q == 1).all()
    lens = qt[:, 3] + qt[:, 1]
    assert (np.diff(lens) <= 0).all()  # longest first
    readers = {a: set() for a in range(C)}
    for t in range(C):
        for a in P[t]:
            readers[int(a)].add(t)
    seen_k = np.zeros(C, np.int64)
    for row0, n, o, nq in kt:
        assert 1 <= n <= 128
        for j in range(n):
            seen_k[row0 + j] += 1
            got = list(ql[o + j:o + nq])
            assert len(got) == len(set(got)) and set(got) == readers[row0 + j]
    assert (seen_k == 1).all()
    assert (np.diff(kt[:, 3]) <= 0).all()
    assert tb["info"]["pairs"] == sum(len(p) for p in P)
    assert list(tb["pos"]) == [len(p) - 1 for p in P]
    return tb


def test_attn_tables_are_the_root_paths():
    m, off, C = np.array([0, 1, 2, 3, 4, 0, 1, 2, 5, 0, 1, 6, 7]), np.array([0, 5, 9, 13]), 8
    tb = _attn_check_tables(m, off, C)
    assert tb["info"]["n_segments"] == 5  # a b | c | d e | f | g h
    rng = np.random.default_rng(11)
    for i in range(6):
        t = trees.random_small_tree(rng, max_segments=9, max_len=150, forest=i % 2 == 1)
        hp = harts.TreePlan(t.tokens, t.offsets, 64)
        _attn_check_tables(np.asarray(hp.maps()[0], np.int64), np.asarray(t.offsets, np.int64), hp.info.C)
    with pytest.raises(harts.HartsError) as e:
        harts.attn_tables(np.array([0, 1, 2, 0, 2]), np.array([0, 3, 5]), 3)
    assert "prefix tree" in str(e.value)
    with pytest.raises(harts.HartsError) as e:
        harts.attn_tables(np.array([0, 1]), np.array([0, 2]), 3)
    assert "no trajectory" in str(e.value)


def test_attn_entry_points_reject_bad_arguments():
    f = harts._lib._attn_fwd
    # unsupported head dims, before any device pointer is touched
    assert f(None, None, None, None, 0, None, 0, 2, 96, 64, 1.0, None, None, None) == -1
    assert f(None, None, None, None, 0, None, 0, 2, 64, 64, 1.0, None, None, None) == 0  # no rows: nothing to do
    assert f(None, None, None, None, 0, None, 4, 2, 64, 64, 1.0, None, None, None) < 0  # rows but no tiles
