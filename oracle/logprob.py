"""Compact -> semantic log-probabilities from their definition -- TEST
INFRASTRUCTURE (see ``oracle/__init__.py``).

For semantic position s with compact row m(s) and target label y_s
(blog section 4.4; paperlayer summary, section 3 "Semantic Preservation"):

    log p_s = x[m(s), y_s] - log sum_v exp(x[m(s), v])

computed in float64 per semantic position (the expanded definition: no
per-row sharing), with the usual max shift inside the log-sum-exp.  The
occurrence count q_c is the number of semantic positions with m(s) = c.

Backward (blog section 4.4, equation 19): for L = sum_s g_s log p_s, every
semantic position forms its own gradient g_s (onehot(y_s) - softmax(x[m(s)]))
and the gradients of all positions that read one compact row are summed into
that row -- a sum of independently formed terms, not a reuse count times one
term, so positions with different labels or weights keep their own parts.
For full-size rows both directions also come in a row-wise form that takes each
row's log-sum-exp (softmax) once with a library routine; those forms are pinned
to the per-position definitions.
"""
from __future__ import annotations

import numpy as np


def logprob(rows_fp64: np.ndarray, row_index: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """``rows_fp64``: float64 logits [R, V]; ``row_index``: for each semantic
    position, the row of ``rows_fp64`` it reads; ``labels``: [S]."""
    row_index = np.asarray(row_index, dtype=np.int64)
    labels = np.asarray(labels, dtype=np.int64)
    out = np.empty(row_index.shape[0], dtype=np.float64)
    step = max(1, (1 << 24) // max(1, rows_fp64.shape[1]))
    for s in range(0, row_index.shape[0], step):
        e = min(row_index.shape[0], s + step)
        x = rows_fp64[row_index[s:e]]
        mx = x.max(axis=1, keepdims=True)
        lse = mx[:, 0] + np.log(np.exp(x - mx).sum(axis=1))
        out[s:e] = x[np.arange(e - s), labels[s:e]] - lse
    return out


def logprob_rowwise(rows_fp64, row_index: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """The same log p_s, with each row's log-sum-exp taken once by a library routine
    (``torch.logsumexp`` over a float64 CPU tensor) and read by every position of that row; for
    full-size rows, where forming it again for each of the S positions would cost S * V
    exponentials.  ``rows_fp64``: float64 logits [R, V] (numpy or CPU torch)."""
    import torch
    x = torch.as_tensor(rows_fp64, dtype=torch.float64)
    lse = torch.logsumexp(x, dim=1)
    ri = torch.as_tensor(np.asarray(row_index, dtype=np.int64))
    lab = torch.as_tensor(np.asarray(labels, dtype=np.int64))
    return (x[ri, lab] - lse[ri]).numpy()


def counts(m: np.ndarray, C: int) -> np.ndarray:
    """q_c = #{s : m(s) = c}."""
    q = np.zeros(C, dtype=np.int64)
    for c in np.asarray(m, dtype=np.int64):
        q[c] += 1
    return q.astype(np.int32)


def logprob_backward(rows_fp64: np.ndarray, row_index: np.ndarray, labels: np.ndarray,
                     dlogp: np.ndarray) -> np.ndarray:
    """dL/dx [R, V] for L = sum_s dlogp[s] * logp[s]: the expanded definition, one semantic
    position at a time (a Python loop: small cases only)."""
    rows = np.asarray(rows_fp64, dtype=np.float64)
    row_index = np.asarray(row_index, dtype=np.int64)
    labels = np.asarray(labels, dtype=np.int64)
    dlogp = np.asarray(dlogp, dtype=np.float64)
    out = np.zeros_like(rows)
    for s in range(row_index.shape[0]):
        x = rows[row_index[s]]
        e = np.exp(x - x.max())
        g = -dlogp[s] * (e / e.sum())
        g[labels[s]] += dlogp[s]
        out[row_index[s]] += g
    return out


def logprob_backward_rowwise(rows_fp64, row_index: np.ndarray, labels: np.ndarray,
                             dlogp: np.ndarray) -> np.ndarray:
    """The same dL/dx [R, V], each row's softmax taken once by a library routine
    (``torch.softmax`` over a float64 CPU tensor): a row's gradient is the sum over its
    positions of g_s onehot(y_s) - g_s softmax(row), and the softmax depends on the row alone,
    so the positions' terms sum to  (sum_s g_s) (-softmax(row))  plus each g_s at its label --
    the per-position sum regrouped, for full-size rows where forming the softmax again for each
    of the S positions would cost S * V exponentials.  ``rows_fp64``: float64 logits [R, V]
    (numpy or CPU torch)."""
    import torch
    x = torch.as_tensor(rows_fp64, dtype=torch.float64)
    ri = np.asarray(row_index, dtype=np.int64)
    g = np.asarray(dlogp, dtype=np.float64)
    weight = np.zeros(x.shape[0], dtype=np.float64)
    np.add.at(weight, ri, g)
    out = torch.softmax(x, dim=1).mul_(-torch.as_tensor(weight)[:, None]).numpy()
    np.add.at(out, (ri, np.asarray(labels, dtype=np.int64)), g)
    return out


def rows_of_map(m: np.ndarray, C: int):
    """The semantic positions of every compact row in increasing order, as CSR offsets [C + 1]
    and positions [S]."""
    m = np.asarray(m, dtype=np.int64)
    off = np.zeros(C + 1, dtype=np.int64)
    pos = []
    for c in range(C):
        mine = [s for s in range(m.shape[0]) if m[s] == c]
        pos.extend(mine)
        off[c + 1] = off[c] + len(mine)
    return off, np.asarray(pos, dtype=np.int64)
