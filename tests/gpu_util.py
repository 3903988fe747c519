"""Helpers for the GPU parity tests: seeded workloads laid out for the device
path (through the C-ABI planner's own map) and for the oracle (through the
oracle planner's own map), compared per generator node."""
from __future__ import annotations

import numpy as np

from synthetic import tensors, trees

TOL = {"fp32": 1e-3, "bf16": 2e-2}


# Smallest normal fp32 number: a reference tensor whose largest magnitude lies below it cannot be
# represented by fp32 state and accumulation at all (steep gates drive handed-off state gradients
# to ~1e-50), so its scale is floored there.
FP32_TINY = float(np.finfo(np.float32).tiny)


def rel_err(x, ref):
    """max |x - ref| / max |ref| per tensor (absolute when ref is exactly zero; the scale floored
    at the smallest normal fp32 number otherwise)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    den = np.abs(ref).max() if ref.size else 0.0
    return float(np.abs(x - ref).max() / (max(den, FP32_TINY) if den > 0 else 1.0)) if ref.size else 0.0


def node_of_row(m: np.ndarray, node_of_pos: np.ndarray, C: int) -> np.ndarray:
    """Generator node of every compact row, from a plan's map m."""
    out = np.full(C, -1, dtype=np.int64)
    out[m] = node_of_pos
    assert (out >= 0).all()
    return out


def device_inputs(feats: tensors.Features, nodes: np.ndarray, device="cuda"):
    import torch
    dt = feats.dtype
    f = feats.gather(nodes)
    out = dict(q=f.q, k=f.k, v=f.v, g=f.g, beta=f.beta)
    if f.do is not None:
        out["do"] = f.do
    return {n: tensors.to_torch(a, dt, device) for n, a in out.items()}


def oracle_feats(feats: tensors.Features):
    return {n: getattr(feats, n).astype(np.float64) for n in ("q", "k", "v", "g", "beta", "do")
            if getattr(feats, n) is not None}


def torch_dtype(dt: str):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


def harts_dtype(dt: str):
    import chunkwise_linear_attention_gated_amd as harts
    return harts.DTYPE_BF16 if dt == "bf16" else harts.DTYPE_FP32
