"""Tree softmax attention over compact rows from its definition -- TEST
INFRASTRUCTURE (see ``oracle/__init__.py``).

The full-attention (MLA) layer of a hybrid model run on compact rows (blog
section 4.3, the MLA paragraph; arXiv summary, section 4, "MLA execution";
Figure C.1(c)): every compact token is projected once, and a branch's queries
read the keys and values of the whole prefix above the branch plus the
branch's own earlier tokens (bottom-right causal alignment: query i of a
branch with h ancestor tokens sees key positions j <= h + i).  Whatever the
packing, the set a compact row t attends over is therefore the root-to-t path
of its trajectory, t included -- the same on every trajectory through t,
since they share t's prefix:

    o[t] = sum_{a in path(t)} softmax_a(scale * <q[t], k[a]>) v[a]

per head.  Computed here row by row in float64 with numpy (small cases).  For
L = sum_t <dout[t], o[t]>, each compact row is one query and the gradients of
its softmax are summed into the rows of its path:

    p = softmax(scale q k^T),  dp = dout v^T,  ds = p (dp - <dout, o>)
    dq[t] += scale ds k,  dk[a] += scale ds q[t],  dv[a] += p dout[t]
"""
from __future__ import annotations

import numpy as np


def parent_rows(m, offsets, C):
    """For every compact row, the row of the token before it on its trajectories (-1 for a
    first token); checks that every trajectory through a row agrees (m is the map of a prefix
    tree) and that every row is on some trajectory."""
    m = np.asarray(m, dtype=np.int64)
    parent = np.full(C, -2, dtype=np.int64)
    depth = np.full(C, -1, dtype=np.int64)
    for tr in range(len(offsets) - 1):
        rows = m[offsets[tr]:offsets[tr + 1]]
        for p in range(len(rows)):
            t = int(rows[p])
            a = int(rows[p - 1]) if p else -1
            if parent[t] == -2:
                parent[t], depth[t] = a, p
            elif parent[t] != a or depth[t] != p:
                raise ValueError(f"row {t} has two different prefixes: not a prefix tree")
    if (parent == -2).any():
        raise ValueError(f"row {int(np.argmax(parent == -2))} is on no trajectory")
    return parent


def path_of(parent, t):
    """Rows of the root-to-t path, root first, t last."""
    out = []
    while t >= 0:
        out.append(t)
        t = int(parent[t])
    return np.array(out[::-1], dtype=np.int64)


def paths(m, offsets, C):
    """For every compact row, the rows of its root-to-row path (root first, the row last)."""
    parent = parent_rows(m, offsets, C)
    return [path_of(parent, t) for t in range(C)]


def row_terms(q, k, v, dout, path, t, h, scale):
    """One query row t of head h over its path (row indices, root first), float64:
    (o [Dv], lse, p [len(path)], ds [len(path)]); ds is None when dout is None.  The
    per-key gradient terms are dk[a] += scale ds[a] q[t] and dv[a] += p[a] dout[t]."""
    qt = np.asarray(q[t, h], dtype=np.float64)
    ka = np.asarray(k[path, h], dtype=np.float64)
    va = np.asarray(v[path, h], dtype=np.float64)
    s = scale * (ka @ qt)
    mx = s.max()
    e = np.exp(s - mx)
    p = e / e.sum()
    o = p @ va
    ds = None
    if dout is not None:
        g = np.asarray(dout[t, h], dtype=np.float64)
        ds = p * (va @ g - g @ o)
    return o, mx + np.log(e.sum()), p, ds


def attention_forward(q, k, v, m, offsets, scale):
    """q, k: [C, H, Dqk]; v: [C, H, Dv]; m: semantic -> compact [S]; offsets [n_traj + 1].
    Returns (o [C, H, Dv], lse [C, H]) in float64; lse is the natural log of the softmax
    denominator, sum_a exp(scale <q[t], k[a]>)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    C, H, _ = q.shape
    P = paths(m, offsets, C)
    o = np.zeros((C, H, v.shape[2]))
    lse = np.zeros((C, H))
    for t in range(C):
        a = P[t]
        for h in range(H):
            s = scale * (k[a, h] @ q[t, h])
            mx = s.max()
            e = np.exp(s - mx)
            o[t, h] = (e @ v[a, h]) / e.sum()
            lse[t, h] = mx + np.log(e.sum())
    return o, lse


def attention_backward(q, k, v, dout, m, offsets, scale):
    """Gradients (dq, dk, dv) of L = sum_t <dout[t], o[t]>, float64, same shapes as q, k, v."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    C, H, _ = q.shape
    P = paths(m, offsets, C)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for t in range(C):
        a = P[t]
        for h in range(H):
            s = scale * (k[a, h] @ q[t, h])
            e = np.exp(s - s.max())
            p = e / e.sum()
            o = p @ v[a, h]
            dp = v[a, h] @ dout[t, h]
            ds = p * (dp - dout[t, h] @ o)
            dq[t, h] += scale * (ds @ k[a, h])
            np.add.at(dk[:, h], a, scale * np.outer(ds, q[t, h]))
            np.add.at(dv[:, h], a, np.outer(p, dout[t, h]))
    return dq, dk, dv
