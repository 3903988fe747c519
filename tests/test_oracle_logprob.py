"""Pins of the float64 log-prob oracle: a constant row, a library
log-softmax, brute-force counts, and the workload generator's invariants."""
import numpy as np
import scipy.special

from oracle import logprob
from synthetic import tensors


def test_constant_row_gives_minus_log_v():
    V = 1000
    x = np.full((3, V), 2.5)
    lp = logprob.logprob(x, np.array([0, 1, 2, 2]), np.array([0, 5, 999, 7]))
    np.testing.assert_allclose(lp, -np.log(V), rtol=0, atol=1e-12)


def test_matches_library_log_softmax():
    rng = np.random.default_rng(0)
    C, V = 17, 513
    x = rng.standard_normal((C, V)) * 2.0
    m = rng.integers(0, C, size=80)
    y = rng.integers(0, V, size=80)
    want = scipy.special.log_softmax(x, axis=1)[m, y]
    np.testing.assert_allclose(logprob.logprob(x, m, y), want, rtol=0, atol=1e-12)


def test_large_logits_are_stable():
    x = np.array([[1000.0, 0.0, -1000.0]])
    lp = logprob.logprob(x, np.array([0, 0]), np.array([0, 1]))
    np.testing.assert_allclose(lp, [0.0, -1000.0], atol=1e-12)


def test_counts_and_generator_invariants():
    w = tensors.logprob_map(C=500, V=4096, seed=1)
    q = logprob.counts(w.m, w.C)
    assert np.array_equal(q, np.bincount(w.m, minlength=w.C))
    assert q.sum() == len(w.m)
    assert (q >= 1).all()
    # labels are distinct within a compact row
    for c in range(50):
        lab = w.labels[w.m == c]
        assert len(np.unique(lab)) == len(lab)
    assert 4.5 < len(w.m) / w.C < 6.8
