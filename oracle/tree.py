"""Expected values for a tree workload from the trajectory-expanded float64
oracle -- TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

The method is a re-ordering of trajectory-wise computation (the pages'
baseline is trajectory-expanded execution; blog sections 5.1 and 6), so the
expected values are defined on expanded trajectories:

* compact output o_c = the output of any semantic copy of c (all copies see
  the same prefix, so they are equal);
* the state handed off at anchor a on a path = the state after a tokens of a
  trajectory through that path;
* with L = sum_c <dO_c, o_c>, dO_c placed on one semantic copy of c (any split
  gives the same gradients, by linearity), the gradient of a compact row's
  features is the sum of the per-position gradients of all its copies;
* the gradient of a handed-off state (blog section 4.3: initial-state
  gradients accumulate back into the call that produced the boundary) is the
  sum over its consumer sequences c of dL_c/dS_a, where L_c keeps only the dO
  of rows in c's subtree.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .planner import Plan
from .recurrent import Trajectories


def _owner_positions(m: np.ndarray, C: int) -> np.ndarray:
    owner = np.full(C, -1, dtype=np.int64)
    for s in range(len(m) - 1, -1, -1):
        owner[m[s]] = s
    return owner


class TreeOracle:
    """``node_of_pos`` maps semantic positions to feature rows (float64
    features ``q, k, v, g`` [R, H, d], ``beta`` [R, H], ``do`` [R, H, dv] when
    a reverse pass is wanted)."""

    def __init__(self, plan: Plan, offsets: np.ndarray, node_of_pos: np.ndarray, feats: Dict[str, np.ndarray]):
        self.plan = plan
        self.offsets = np.asarray(offsets, dtype=np.int64)
        self.node_of_pos = np.asarray(node_of_pos, dtype=np.int64)
        self.F = feats
        self.owner = _owner_positions(plan.m, plan.C)
        self.traj_of_pos = np.repeat(np.arange(len(offsets) - 1), np.diff(self.offsets))
        # feature row of every compact row
        self.feat_row = self.node_of_pos[self.owner]

    def _traj(self, which: Sequence[int]) -> Trajectories:
        rows = [self.node_of_pos[self.offsets[x]:self.offsets[x + 1]] for x in which]
        F = self.F
        return Trajectories(rows, F["q"], F["k"], F["v"], F["g"], F["beta"])

    def forward(self, which: Optional[Sequence[int]] = None, nthreads: int = 0):
        """Compact outputs for every row owned by a selected trajectory (NaN
        elsewhere) and every slot whose producer row lies on a selected
        trajectory (NaN elsewhere)."""
        plan = self.plan
        which = list(range(len(self.offsets) - 1)) if which is None else list(which)
        caps, cap_slot = [], []
        for sl, key in enumerate(plan.slot_row):
            s = self.owner[key]
            x = int(self.traj_of_pos[s])
            if x in which:
                caps.append((which.index(x), int(s - self.offsets[x]) + 1))
                cap_slot.append(sl)
        tr = self._traj(which)
        o_pos, st = tr.forward(captures=caps, nthreads=nthreads)
        H, dv = o_pos.shape[1:]
        o = np.full((plan.C, H, dv), np.nan)
        base = 0
        for i, x in enumerate(which):
            L = int(self.offsets[x + 1] - self.offsets[x])
            o[plan.m[self.offsets[x]:self.offsets[x + 1]]] = o_pos[base:base + L]
            base += L
        slots = np.full((plan.n_slots, H, self.F["k"].shape[2], dv), np.nan)
        for j, sl in enumerate(cap_slot):
            slots[sl] = st[j]
        return o, slots

    def backward(self, do_compact: np.ndarray, nthreads: int = 0, slot_grads: bool = True):
        """Compact gradients (all trajectories) and slot gradients."""
        plan = self.plan
        n = len(self.offsets) - 1
        tr = self._traj(range(n))
        dO = np.zeros((plan.S,) + do_compact.shape[1:])
        dO[self.owner] = do_compact
        res = tr.backward(dO, nthreads=nthreads)
        out = {}
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            acc = np.zeros((plan.C,) + res[name].shape[1:])
            np.add.at(acc, plan.m, res[name])
            out[name] = acc
        if slot_grads:
            out["dslots"] = self.slot_gradients(dO, nthreads=nthreads)
        return out

    def slot_gradients(self, dO_pos: np.ndarray, nthreads: int = 0) -> np.ndarray:
        plan = self.plan
        H, dk, dv = self.F["q"].shape[1], self.F["q"].shape[2], self.F["v"].shape[2]
        dslots = np.zeros((plan.n_slots, H, dk, dv))
        seg = plan.segments
        node_row = np.empty(plan.C, dtype=np.int64)
        node_row[plan.trie.m_node] = plan.m
        for sp in plan.seqs:
            if sp.init_slot < 0:
                continue
            s_v = seg.start[sp.head]
            head_row = node_row[seg.nodes[sp.head][0]]
            xs = [x for x in range(len(self.offsets) - 1)
                  if self.offsets[x + 1] - self.offsets[x] > s_v and plan.m[self.offsets[x] + s_v] == head_row]
            rows = [self.node_of_pos[self.offsets[x]:self.offsets[x + 1]] for x in xs]
            F = self.F
            tr = Trajectories(rows, F["q"], F["k"], F["v"], F["g"], F["beta"])
            d = np.concatenate([dO_pos[self.offsets[x]:self.offsets[x + 1]] for x in xs]).copy()
            base = 0
            for x in xs:
                d[base:base + s_v] = 0.0  # keep only the consumer subtree's rows
                base += int(self.offsets[x + 1] - self.offsets[x])
            res = tr.backward(d, captures=[(i, sp.start) for i in range(len(xs))], nthreads=nthreads)
            dslots[sp.init_slot] += res["lam"].sum(axis=0)
        return dslots
