"""Tree causal convolution from its expanded definition -- TEST INFRASTRUCTURE
(see ``oracle/__init__.py``).

The KDA layer's depthwise causal convolution over compact rows (blog section
4.3): the window of a token is the previous w - 1 tokens of its own
trajectory -- the real ancestors, whichever segment or round holds them --
and nothing before the trajectory's first token:

    out[t, c] = sum_{j=0}^{w-1} weight[c, j] * x[t_{-j}, c]

where t_{-j} is the token j places before t on a trajectory through t (every
trajectory through t agrees, since they share t's prefix).  Computed here one
trajectory at a time in float64 (plain loops: small cases only); for the
gradient of L = sum_t <dout[t], out[t]>, each compact row's output is taken
from one trajectory through it and differentiated term by term.
"""
from __future__ import annotations

import numpy as np


def _first_positions(m, offsets):
    """For every compact row, (trajectory, position) of one semantic position reading it."""
    first = {}
    for tr in range(len(offsets) - 1):
        for p in range(offsets[tr + 1] - offsets[tr]):
            first.setdefault(int(m[offsets[tr] + p]), (tr, p))
    return first


def conv_forward(x, weight, m, offsets):
    """x: float [C, Ch] compact rows; weight: [Ch, w]; m: semantic -> compact [S];
    offsets: trajectory offsets [n_traj + 1].  Returns out [C, Ch] (float64), from every
    trajectory (and checks that trajectories sharing a row agree on it)."""
    x = np.asarray(x, dtype=np.float64)
    wgt = np.asarray(weight, dtype=np.float64)
    m = np.asarray(m, dtype=np.int64)
    C, Ch = x.shape
    w = wgt.shape[1]
    out = np.full((C, Ch), np.nan)
    for tr in range(len(offsets) - 1):
        rows = m[offsets[tr]:offsets[tr + 1]]
        for p in range(rows.shape[0]):
            acc = np.zeros(Ch)
            for j in range(w):
                if p - j >= 0:
                    acc += wgt[:, j] * x[rows[p - j]]
            t = rows[p]
            if np.isnan(out[t, 0]):
                out[t] = acc
            else:
                assert np.array_equal(out[t], acc), "trajectories disagree on a shared row"
    return out


def conv_backward(x, weight, m, offsets, dout):
    """Gradients (dx [C, Ch], dweight [Ch, w]) of L = sum_t <dout[t], out[t]>."""
    x = np.asarray(x, dtype=np.float64)
    wgt = np.asarray(weight, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    m = np.asarray(m, dtype=np.int64)
    C, Ch = x.shape
    w = wgt.shape[1]
    dx = np.zeros((C, Ch))
    dw = np.zeros((Ch, w))
    for t, (tr, p) in sorted(_first_positions(m, offsets).items()):
        rows = m[offsets[tr]:offsets[tr + 1]]
        for j in range(w):
            if p - j >= 0:
                s = rows[p - j]
                dx[s] += wgt[:, j] * dout[t]
                dw[:, j] += dout[t] * x[s]
    return dx, dw
