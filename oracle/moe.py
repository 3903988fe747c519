"""Multiplicity-weighted MoE router statistics from their expanded definitions --
TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Compact rows are routed once (blog section 4.3, MoE paragraph; arXiv summary,
section 4, "MoE execution"), and the multiplicity q_c -- the number of semantic
positions mapped to compact row c, sum_c q_c = S -- restores every training
weight (blog section 4.4; Figure C.1(d)): the router z-loss takes q_c as the
row's token weight; the load-balance loss weights the routing probability mass
and the top-k assignment counts by q_c; the expert-bias update uses the same
weighted counts.  Multiplicity changes no routing decision.

Per compact row c with router logits z[c] over E experts and expert bias b
(float64 here):

    p[c]    = softmax(z[c]);  lse_c = log sum_e exp(z[c, e])
    top_c   = the k experts with the largest p[c, e] + b[e] (ties: lower index)
    n_e     = sum_c q_c [e in top_c]              (weighted assignment counts)
    P_e     = sum_c q_c p[c, e]                   (weighted probability mass)
    L_z     = (1 / S) sum_c q_c lse_c^2
    L_aux   = E / (k S^2) sum_e n_e P_e
    b'_e    = b_e + gamma * sign(mean_j n_j - n_e)

which are the per-position definitions summed over the S semantic positions (a
position reads the row it maps to).  Gradient of z_coef L_z + aux_coef L_aux
with respect to z (the counts are piecewise constant):

    dz[c, e] = z_coef 2 q_c lse_c p[c, e] / S
             + aux_coef E / (k S^2) q_c p[c, e] (n_e - sum_j n_j p[c, j])
"""
from __future__ import annotations

import numpy as np


def route(z, bias, k):
    """(p [C, E], lse [C], top [C, k] int64) in float64; top in decreasing score order."""
    z = np.asarray(z, dtype=np.float64)
    mx = z.max(axis=1, keepdims=True)
    e = np.exp(z - mx)
    p = e / e.sum(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(e.sum(axis=1))
    s = p + np.asarray(bias, dtype=np.float64)[None, :]
    top = np.argsort(-s, axis=1, kind="stable")[:, :k]
    return p, lse, top


def statistics(z, bias, q, k, S):
    """dict: counts n [E] (int64), mass P [E], L_z, L_aux, top [C, k], lse [C]."""
    p, lse, top = route(z, bias, k)
    C, E = p.shape
    q = np.asarray(q, dtype=np.int64)
    n = np.zeros(E, dtype=np.int64)
    for c in range(C):
        n[top[c]] += q[c]
    P = (q[:, None] * p).sum(axis=0)
    Lz = float((q * lse ** 2).sum() / S)
    Laux = float(E / (k * S * S) * (n * P).sum())
    return {"counts": n, "mass": P, "L_z": Lz, "L_aux": Laux, "top": top, "lse": lse}


def grad(z, bias, q, k, S, z_coef, aux_coef):
    """dz [C, E] float64 of z_coef L_z + aux_coef L_aux (counts held fixed)."""
    p, lse, _ = route(z, bias, k)
    st = statistics(z, bias, q, k, S)
    C, E = p.shape
    q = np.asarray(q, dtype=np.float64)[:, None]
    n = st["counts"].astype(np.float64)[None, :]
    nbar = (p * n).sum(axis=1, keepdims=True)
    return z_coef * 2.0 * q * lse[:, None] * p / S + aux_coef * E / (k * S * S) * q * p * (n - nbar)


def bias_update(bias, counts, gamma):
    counts = np.asarray(counts, dtype=np.float64)
    return np.asarray(bias, dtype=np.float64) + gamma * np.sign(counts.mean() - counts)
