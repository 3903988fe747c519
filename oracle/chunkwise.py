"""Float64 chunkwise form of the gated delta rule, and tree execution with
bounded replay -- TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Used only to check the oracle against itself and against the pages' claims:
the chunkwise-parallel form (fixed chunk B, parallel inside a chunk, state
passed between chunks -- blog section 1.2 and glossary) equals the recurrent
form; a tree executed round by round, each sequence starting from a
chunk-boundary state and replaying the < B ancestor tokens [a(p), p)
(blog section 4.2, "replay"), equals trajectory-wise chunked execution
bit for bit; starting a side branch from its parent's end state instead (the
no-replay ablation, blog section 5.3) does not.

Per chunk of l tokens with initial state S0 (per head), G_r the inclusive
cumulative sum of g over the chunk:

    A_ij = sum_c k_ic k_jc exp(G_ic - G_jc)  for i > j   (0 otherwise)
    M_ij = sum_c q_ic k_jc exp(G_ic - G_jc)  for i >= j
    T    = (I + diag(beta) A)^{-1} diag(beta)
    U    = T (V - (K * exp(G)) S0)
    O    = (Q * exp(G)) S0 + M U
    S_l  = diag(exp(G_l)) S0 + (K * exp(G_l - G))^T U

The pairwise exponentials are formed directly (no factorisation), which is
the plain definition.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np
import scipy.linalg

from .planner import Plan


def chunk_step(q, k, v, g, beta, S0):
    """One chunk.  q, k, g: [l, H, dk]; v: [l, H, dv]; beta: [l, H];
    S0: [H, dk, dv].  Returns (O [l, H, dv], S_l [H, dk, dv])."""
    l, H, dk = k.shape
    dv = v.shape[2]
    O = np.zeros((l, H, dv))
    S1 = np.zeros((H, dk, dv))
    G = np.cumsum(g, axis=0)
    tri_s = np.tril(np.ones((l, l)), -1)
    tri_i = np.tril(np.ones((l, l)), 0)
    for h in range(H):
        Gh = G[:, h, :]
        D = np.exp(Gh[:, None, :] - Gh[None, :, :]) * (tri_i[:, :, None] > 0)  # [i, j, c], i >= j
        A = np.einsum("ic,jc,ijc->ij", k[:, h], k[:, h], D) * tri_s
        M = np.einsum("ic,jc,ijc->ij", q[:, h], k[:, h], D) * tri_i
        L = np.eye(l) + beta[:, h][:, None] * A
        T = scipy.linalg.solve_triangular(L, np.diag(beta[:, h]), lower=True)
        E = np.exp(Gh)
        U = T @ (v[:, h] - (k[:, h] * E) @ S0[h])
        O[:, h] = (q[:, h] * E) @ S0[h] + M @ U
        S1[h] = E[-1][:, None] * S0[h] + (k[:, h] * np.exp(Gh[-1][None, :] - Gh)).T @ U
    return O, S1


def run_sequence(q, k, v, g, beta, S0, B: int, boundaries: bool = False):
    """Chunks of B tokens from the first token.  Returns O [L, H, dv], the final
    state, and (optionally) the state after every multiple of B in (0, L]."""
    L = k.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((L, k.shape[1], v.shape[2]))
    states = []
    for s in range(0, L, B):
        e = min(L, s + B)
        O[s:e], S = chunk_step(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], S)
        if boundaries and e - s == B:
            states.append(S.copy())
    return O, S, states


def run_tree_replay(plan: Plan, F: Dict[str, np.ndarray]):
    """Round-by-round tree execution with bounded replay.

    ``F`` holds float64 features on compact rows (``q, k, v, g`` [C, H, d],
    ``beta`` [C, H]).  Each sequence's virtual stream is its replay rows then
    its own rows, chunked from its anchor; it starts from the zero state or its
    slot, writes outputs for its own rows only, and stores the boundary states
    it emits into slots.  Returns (o [C, H, dv], slots [n_slots, H, dk, dv])."""
    C, H, dk = F["k"].shape
    dv = F["v"].shape[2]
    B = plan.B
    o = np.full((C, H, dv), np.nan)
    slots = np.full((plan.n_slots, H, dk, dv), np.nan)
    for r in range(1, plan.n_rounds + 1):
        ready = slots.copy()  # states produced inside a call are usable only after it returns
        for i in plan.round_seqs(r):
            sp = plan.seqs[i]
            rows = np.asarray(sp.replay_rows + sp.own_rows, dtype=np.int64)
            S = np.zeros((H, dk, dv)) if sp.init_slot < 0 else ready[sp.init_slot]
            assert not np.isnan(S).any(), "slot used before it was produced"
            emits = dict(sp.emits)
            L = len(rows)
            for n, s in enumerate(range(0, L, B)):
                e = min(L, s + B)
                rr = rows[s:e]
                O, S = chunk_step(F["q"][rr], F["k"][rr], F["v"][rr], F["g"][rr], F["beta"][rr], S)
                for t in range(s, e):
                    if t >= len(sp.replay_rows):
                        o[rows[t]] = O[t - s]
                if (n + 1) in emits:
                    slots[emits[n + 1]] = S
    return o, slots


def run_trajectories_chunked(plan: Plan, F: Dict[str, np.ndarray], offsets: np.ndarray, B: int,
                             which: Optional[List[int]] = None):
    """Trajectory-wise chunked execution: every expanded trajectory from the
    zero state, chunks aligned at its first token.  Returns per-position
    outputs for the selected trajectories (dict traj -> [L, H, dv])."""
    out = {}
    H, dk = F["k"].shape[1:]
    dv = F["v"].shape[2]
    for x in (which if which is not None else range(len(offsets) - 1)):
        rows = plan.m[offsets[x]:offsets[x + 1]]
        O, _, _ = run_sequence(F["q"][rows], F["k"][rows], F["v"][rows], F["g"][rows], F["beta"][rows],
                               np.zeros((H, dk, dv)), B)
        out[x] = O
    return out


def run_tree_no_replay(plan: Plan, F: Dict[str, np.ndarray]):
    """The no-replay ablation: a side branch starts from its parent's exact
    state at the fork (no realignment to the chunk phase), with chunks counted
    from the fork.  Returns o [C, H, dv]."""
    C, H, dk = F["k"].shape
    dv = F["v"].shape[2]
    seg = plan.segments
    B = plan.B
    # state at the end of every segment along its path, computed depth first
    o = np.full((C, H, dv), np.nan)
    node_row = np.empty(plan.C, dtype=np.int64)
    node_row[plan.trie.m_node] = plan.m
    end_state = {}
    for v in seg.preorder:
        p = seg.parent[v]
        S0 = np.zeros((H, dk, dv)) if p < 0 else end_state[p]
        rows = node_row[np.asarray(seg.nodes[v])]
        O, S, _ = run_sequence(F["q"][rows], F["k"][rows], F["v"][rows], F["g"][rows], F["beta"][rows], S0, B)
        o[rows] = O
        end_state[v] = S
    return o
