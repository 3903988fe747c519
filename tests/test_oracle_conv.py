"""Pins of the float64 tree-convolution oracle: a single trajectory against a
library convolution, a shared prefix giving the same row values on every
trajectory, and central finite differences for both gradients."""
import numpy as np

from oracle import conv


def _tree():
    # three trajectories: [a b c d e] [a b c f] [a b g h i j]; rows: a=0 b=1 c=2 d=3 e=4 f=5 g=6 h=7 i=8 j=9
    m = np.array([0, 1, 2, 3, 4, 0, 1, 2, 5, 0, 1, 6, 7, 8, 9])
    off = np.array([0, 5, 9, 15])
    return m, off, 10


def test_single_trajectory_is_a_causal_convolution():
    rng = np.random.default_rng(0)
    L, Ch, w = 12, 3, 4
    x = rng.standard_normal((L, Ch))
    wgt = rng.standard_normal((Ch, w))
    out = conv.conv_forward(x, wgt, np.arange(L), np.array([0, L]))
    for c in range(Ch):
        np.testing.assert_allclose(out[:, c], np.convolve(x[:, c], wgt[c])[:L], rtol=0, atol=1e-12)


def test_rows_after_a_fork_see_the_ancestors():
    m, off, C = _tree()
    rng = np.random.default_rng(1)
    x = rng.standard_normal((C, 2))
    wgt = rng.standard_normal((2, 3))
    out = conv.conv_forward(x, wgt, m, off)
    # row g (6) follows a, b on its trajectory: window (g, b, a)
    np.testing.assert_allclose(out[6], wgt[:, 0] * x[6] + wgt[:, 1] * x[1] + wgt[:, 2] * x[0], atol=1e-12)
    # row f (5) follows c, b: window (f, c, b)
    np.testing.assert_allclose(out[5], wgt[:, 0] * x[5] + wgt[:, 1] * x[2] + wgt[:, 2] * x[1], atol=1e-12)
    # the first token sees only itself
    np.testing.assert_allclose(out[0], wgt[:, 0] * x[0], atol=1e-12)


def test_gradients_match_finite_differences():
    m, off, C = _tree()
    rng = np.random.default_rng(2)
    Ch, w = 2, 4
    x = rng.standard_normal((C, Ch))
    wgt = rng.standard_normal((Ch, w))
    dout = rng.standard_normal((C, Ch))
    dx, dw = conv.conv_backward(x, wgt, m, off, dout)
    loss = lambda xx, ww: float((conv.conv_forward(xx, ww, m, off) * dout).sum())  # noqa: E731
    h = 1e-6
    for t in range(C):
        for c in range(Ch):
            xp, xm = x.copy(), x.copy()
            xp[t, c] += h
            xm[t, c] -= h
            assert abs(dx[t, c] - (loss(xp, wgt) - loss(xm, wgt)) / (2 * h)) < 1e-7
    for c in range(Ch):
        for j in range(w):
            wp, wm = wgt.copy(), wgt.copy()
            wp[c, j] += h
            wm[c, j] -= h
            assert abs(dw[c, j] - (loss(x, wp) - loss(x, wm)) / (2 * h)) < 1e-7
