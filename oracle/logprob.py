"""Compact -> semantic log-probabilities from their definition -- TEST
INFRASTRUCTURE (see ``oracle/__init__.py``).

For semantic position s with compact row m(s) and target label y_s
(blog section 4.4; paperlayer summary, section 3 "Semantic Preservation"):

    log p_s = x[m(s), y_s] - log sum_v exp(x[m(s), v])

computed in float64 per semantic position (the expanded definition: no
per-row sharing), with the usual max shift inside the log-sum-exp.  The
occurrence count q_c is the number of semantic positions with m(s) = c.
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


def counts(m: np.ndarray, C: int) -> np.ndarray:
    """q_c = #{s : m(s) = c}."""
    q = np.zeros(C, dtype=np.int64)
    for c in np.asarray(m, dtype=np.int64):
        q[c] += 1
    return q.astype(np.int32)
