"""Seeded per-node features and the log-prob workload.

Distributions (the gated-delta workloads of the pages' evaluation setting,
synthetic stand-ins for the Ling models' activations):

* q, k ~ N(0, 1), then scaled to unit L2 norm per (token, head);
* v ~ N(0, 1);
* g = -softplus(N(0, 1)) per channel (a log-decay, always <= 0);
* beta = sigmoid(N(0, 1)) per (token, head);
* dO ~ N(0, 1) per compact token (the upstream gradient of o).

Values are drawn in float64 per node (generator node order, tensor by tensor
in the order q, k, v, g, beta), then rounded to the working dtype: for
``"bf16"`` with round-to-nearest-even (normalisation happens before rounding,
so norms are only close to 1).  Arrays are returned as float32 holding
exactly representable values; :func:`to_torch` makes device tensors of the
working dtype without further rounding.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to the nearest bfloat16 (ties to even);
    returns float32 holding the rounded values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _normal(rng: np.random.Generator, shape, chunk_rows: int = 1 << 14) -> np.ndarray:
    # drawn in blocks of rows so large workloads stay within memory
    out = np.empty(shape, dtype=np.float32)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        out[s:e] = rng.standard_normal((e - s,) + tuple(shape[1:]))
    return out


@dataclass
class Features:
    q: np.ndarray      # [n_nodes, H, dk]
    k: np.ndarray      # [n_nodes, H, dk]
    v: np.ndarray      # [n_nodes, H, dv]
    g: np.ndarray      # [n_nodes, H, dk]
    beta: np.ndarray   # [n_nodes, H]
    do: Optional[np.ndarray]  # [n_nodes, H, dv]
    dtype: str

    def gather(self, nodes: np.ndarray) -> "Features":
        nodes = np.asarray(nodes)
        return Features(self.q[nodes], self.k[nodes], self.v[nodes], self.g[nodes], self.beta[nodes],
                        None if self.do is None else self.do[nodes], self.dtype)


def draw_features(n_nodes: int, H: int, dk: int, dv: int, seed: int = 0, dtype: str = "bf16",
                  with_do: bool = True) -> Features:
    rng = np.random.default_rng(np.random.PCG64([seed, 0xF00D]))

    def unit(x):
        x64 = x.astype(np.float64)
        n = np.sqrt((x64 * x64).sum(-1, keepdims=True))
        return (x64 / np.maximum(n, 1e-30)).astype(np.float32)

    q = _round(unit(_normal(rng, (n_nodes, H, dk))), dtype)
    k = _round(unit(_normal(rng, (n_nodes, H, dk))), dtype)
    v = _round(_normal(rng, (n_nodes, H, dv)), dtype)
    x = _normal(rng, (n_nodes, H, dk)).astype(np.float64)
    g = _round(-np.logaddexp(0.0, x), dtype)
    del x
    b = rng.standard_normal((n_nodes, H))
    beta = _round(1.0 / (1.0 + np.exp(-b)), dtype)
    do = _round(_normal(rng, (n_nodes, H, dv)), dtype) if with_do else None
    return Features(q, k, v, g, beta, do, dtype)


def initial_states(n: int, H: int, dk: int, dv: int, seed: int = 0, std: float = 0.1) -> np.ndarray:
    """fp32 N(0, std^2) initial states [n, H, dk, dv]."""
    rng = np.random.default_rng(np.random.PCG64([seed, 0x1717]))
    return (_normal(rng, (n, H, dk, dv)) * np.float32(std)).astype(np.float32)


# ---------------------------------------------------------------- log-prob workload

@dataclass
class LogprobWorkload:
    C: int
    V: int
    m: np.ndarray       # int64 [S]  semantic position -> compact row
    labels: np.ndarray  # int32 [S]  target token per semantic position


def logprob_map(C: int, V: int, seed: int = 0, mean_mult: float = 5.6) -> LogprobWorkload:
    """Multiplicities 1 + Geometric (mean ``mean_mult`` in total, so every row
    is used), semantic positions a seeded shuffle of the resulting multiset,
    labels uniform over V and pairwise distinct within a row."""
    rng = np.random.default_rng(np.random.PCG64([seed, 0x4242]))
    mult = rng.geometric(1.0 / mean_mult, size=C).astype(np.int64)
    mult = np.minimum(mult, V)
    rows = np.repeat(np.arange(C, dtype=np.int64), mult)
    labels_by_row = np.empty(rows.shape[0], dtype=np.int64)
    pos = 0
    for c in range(C):
        q = int(mult[c])
        lab = rng.integers(0, V, size=q)
        while len(np.unique(lab)) < q:
            u = np.unique(lab)
            lab = np.concatenate([u, rng.integers(0, V, size=q - len(u))])
        labels_by_row[pos:pos + q] = lab
        pos += q
    perm = rng.permutation(rows.shape[0])
    return LogprobWorkload(C=C, V=V, m=rows[perm].copy(), labels=labels_by_row[perm].astype(np.int32))


def logits_torch(C: int, V: int, seed: int = 0, device: str = "cpu", std: float = 2.0, dtype=None):
    """Logits N(0, std^2) [C, V] drawn by torch's generator on ``device``
    (bfloat16 by default)."""
    import torch
    dtype = dtype or torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty((C, V), dtype=dtype, device=device)
    rows = max(1, (1 << 26) // V)
    for s in range(0, C, rows):
        e = min(C, s + rows)
        out[s:e] = (torch.randn((e - s, V), generator=gen, device=device, dtype=torch.float32) * std).to(dtype)
    return out


def to_torch(x: np.ndarray, dtype: str, device="cpu"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(device)
