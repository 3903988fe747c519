"""Pins of the float64 log-prob oracle: a constant row, a library
log-softmax, brute-force counts, and the workload generator's invariants;
for its backward, central finite differences of the forward, the zero row
sum, a library cross-entropy gradient and the additivity of repeated
positions."""
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


def test_rowwise_form_matches_the_per_position_definition_and_library():
    rng = np.random.default_rng(3)
    C, V = 23, 777
    x = rng.standard_normal((C, V)) * 3.0
    x[5] = 1.25  # a constant row: exactly -ln V
    m = rng.integers(0, C, size=200)
    m[:4] = 5
    y = rng.integers(0, V, size=200)
    got = logprob.logprob_rowwise(x, m, y)
    np.testing.assert_allclose(got, logprob.logprob(x, m, y), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got, scipy.special.log_softmax(x, axis=1)[m, y], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[:4], -np.log(V), rtol=0, atol=1e-12)
    big = np.array([[1000.0, 0.0, -1000.0]])
    np.testing.assert_allclose(logprob.logprob_rowwise(big, [0, 0], [0, 2]), [0.0, -2000.0], atol=1e-12)


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


def _fd_grad(x, m, y, w, c, v, h=1e-6):
    xp, xm = x.copy(), x.copy()
    xp[c, v] += h
    xm[c, v] -= h
    return (w @ logprob.logprob(xp, m, y) - w @ logprob.logprob(xm, m, y)) / (2 * h)


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(5)
    C, V, S = 4, 37, 11
    x = rng.standard_normal((C, V)) * 1.5
    m = rng.integers(0, C, size=S)
    y = rng.integers(0, V, size=S)
    y[3], m[3] = y[2], m[2]  # a repeated (row, label) pair
    w = rng.standard_normal(S)
    g = logprob.logprob_backward(x, m, y, w)
    for c in range(C):
        for v in list(rng.integers(0, V, size=6)) + [int(y[s]) for s in range(S) if m[s] == c]:
            assert abs(g[c, v] - _fd_grad(x, m, y, w, c, v)) < 1e-7


def test_backward_rows_sum_to_zero_and_unread_rows_are_zero():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((6, 50))
    m = np.array([0, 0, 2, 3, 3, 3])
    y = np.array([1, 1, 7, 0, 49, 2])
    g = logprob.logprob_backward(x, m, y, rng.standard_normal(6))
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-12)
    assert not g[[1, 4, 5]].any()


def test_backward_single_positions_match_library_cross_entropy():
    torch = __import__("pytest").importorskip("torch")
    rng = np.random.default_rng(7)
    C, V = 5, 64
    x = rng.standard_normal((C, V))
    y = rng.integers(0, V, size=C)
    xt = torch.tensor(x, requires_grad=True)
    torch.nn.functional.cross_entropy(xt, torch.tensor(y), reduction="sum").backward()
    # L = sum log p = -cross entropy: the gradient is the negated library one
    np.testing.assert_allclose(logprob.logprob_backward(x, np.arange(C), y, np.ones(C)), -xt.grad.numpy(),
                               rtol=0, atol=1e-12)


def test_backward_repeated_positions_add():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 20))
    one = logprob.logprob_backward(x, np.array([1]), np.array([4]), np.array([0.7]))
    two = logprob.logprob_backward(x, np.array([1, 1]), np.array([4, 4]), np.array([0.7, 0.7]))
    np.testing.assert_allclose(two, 2 * one, rtol=0, atol=1e-14)
    mixed = logprob.logprob_backward(x, np.array([1, 1]), np.array([4, 9]), np.array([0.7, -0.2]))
    np.testing.assert_allclose(mixed, one + logprob.logprob_backward(x, np.array([1]), np.array([9]), np.array([-0.2])),
                               rtol=0, atol=1e-14)


def test_rowwise_backward_matches_the_per_position_definition_and_autograd():
    torch = __import__("pytest").importorskip("torch")
    rng = np.random.default_rng(10)
    C, V, S = 9, 53, 40
    x = rng.standard_normal((C, V)) * 2.0
    m = rng.integers(0, C - 2, size=S)  # the last two rows are read by no position
    y = rng.integers(0, V, size=S)
    y[5], m[5] = y[4], m[4]  # a repeated (row, label) pair
    w = rng.standard_normal(S)
    g = logprob.logprob_backward_rowwise(x, m, y, w)
    np.testing.assert_allclose(g, logprob.logprob_backward(x, m, y, w), rtol=0, atol=1e-13)
    assert not g[C - 2:].any()
    xt = torch.tensor(x, requires_grad=True)
    lp = torch.log_softmax(xt, dim=1)[torch.tensor(m), torch.tensor(y)]
    (lp * torch.tensor(w)).sum().backward()
    np.testing.assert_allclose(g, xt.grad.numpy(), rtol=0, atol=1e-13)
    for c, v in [(int(m[0]), int(y[0])), (int(m[7]), 3), (0, 11)]:
        assert abs(g[c, v] - _fd_grad(x, m, y, w, c, v)) < 1e-7


def test_rows_of_map_is_the_stable_inverse():
    rng = np.random.default_rng(9)
    m = rng.integers(0, 7, size=40)
    off, pos = logprob.rows_of_map(m, 9)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(m, minlength=9))]))
    assert np.array_equal(pos, np.argsort(m, kind="stable"))
