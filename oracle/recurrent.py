"""ctypes front end of the float64 token-recurrent oracle (``recurrent.c``).

TEST INFRASTRUCTURE: see ``oracle/__init__.py``.  Builds ``_recurrent.so``
with gcc (plain ISO float64, no fast-math) on first use when it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_recurrent.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle library with gcc."""
    src = os.path.join(_HERE, "recurrent.c")
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _TrajIn(ctypes.Structure):
    _fields_ = [("n_traj", ctypes.c_int64), ("offsets", ctypes.c_void_p), ("nodes", ctypes.c_void_p),
                ("H", ctypes.c_int), ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("S0", ctypes.c_void_p)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        _lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        _lib.oracle_fwd.argtypes = [ctypes.POINTER(_TrajIn), P, P, P, P, P, ctypes.c_int]
        _lib.oracle_bwd.argtypes = [ctypes.POINTER(_TrajIn), P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        _lib.oracle_fwd.restype = ctypes.c_int
        _lib.oracle_bwd.restype = ctypes.c_int
        _lib.oracle_num_threads.restype = ctypes.c_int
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


class Trajectories:
    """Trajectories as lists of feature-row indices, plus float64 features
    ``q, k, g`` [R, H, dk], ``v`` [R, H, dv], ``beta`` [R, H]."""

    def __init__(self, rows: Sequence[np.ndarray], q, k, v, g, beta, S0: Optional[np.ndarray] = None):
        self.offsets = np.zeros(len(rows) + 1, dtype=np.int64)
        self.offsets[1:] = np.cumsum([len(r) for r in rows])
        self.nodes = np.ascontiguousarray(np.concatenate([np.asarray(r, dtype=np.int64) for r in rows])
                                          if rows else np.zeros(0, np.int64))
        f = lambda a: np.ascontiguousarray(a, dtype=np.float64)
        self.q, self.k, self.v, self.g, self.beta = f(q), f(k), f(v), f(g), f(beta)
        self.H, self.dk = self.q.shape[1], self.q.shape[2]
        self.dv = self.v.shape[2]
        self.S0 = None if S0 is None else f(S0)
        self._keep = None

    @property
    def P(self) -> int:
        return int(self.offsets[-1])

    def _struct(self) -> _TrajIn:
        return _TrajIn(len(self.offsets) - 1, _p(self.offsets), _p(self.nodes), self.H, self.dk, self.dv,
                       _p(self.q), _p(self.k), _p(self.v), _p(self.g), _p(self.beta), _p(self.S0))

    def _caps(self, captures):
        if not captures:
            return None, None, None, 0
        n = len(self.offsets) - 1
        order = sorted(range(len(captures)), key=lambda i: captures[i][0])
        cap_off = np.zeros(n + 1, dtype=np.int64)
        for (x, _) in captures:
            cap_off[x + 1] += 1
        cap_off = np.cumsum(cap_off).astype(np.int64)
        cap_pos = np.asarray([captures[i][1] for i in order], dtype=np.int64)
        cap_out = np.asarray(order, dtype=np.int64)
        return cap_off, cap_pos, cap_out, len(captures)

    def forward(self, captures: Sequence[Tuple[int, int]] = (), nthreads: int = 0):
        """o per position [P, H, dv]; states after ``a`` tokens of trajectory
        ``x`` for each capture (x, a), [n_cap, H, dk, dv]."""
        lib = _load()
        o = np.zeros((self.P, self.H, self.dv))
        cap_off, cap_pos, cap_out, ncap = self._caps(captures)
        st = np.zeros((ncap, self.H, self.dk, self.dv))
        s = self._struct()
        rc = lib.oracle_fwd(ctypes.byref(s), _p(o), _p(cap_off), _p(cap_pos), _p(cap_out), _p(st),
                            nthreads or default_threads())
        if rc:
            raise MemoryError("oracle_fwd")
        return o, st

    def backward(self, dO: np.ndarray, captures: Sequence[Tuple[int, int]] = (), nthreads: int = 0):
        """Gradients of L = sum <dO, o> per position, dS0 per trajectory, and
        lambda = dL/dS_a for each capture (x, a)."""
        lib = _load()
        dO = np.ascontiguousarray(dO, dtype=np.float64)
        P, H, dk, dv = self.P, self.H, self.dk, self.dv
        dq = np.zeros((P, H, dk)); dk_ = np.zeros((P, H, dk)); dv_ = np.zeros((P, H, dv))
        dg = np.zeros((P, H, dk)); db = np.zeros((P, H))
        dS0 = np.zeros((len(self.offsets) - 1, H, dk, dv))
        cap_off, cap_pos, cap_out, ncap = self._caps(captures)
        lam = np.zeros((ncap, H, dk, dv))
        s = self._struct()
        rc = lib.oracle_bwd(ctypes.byref(s), _p(dO), _p(dq), _p(dk_), _p(dv_), _p(dg), _p(db), _p(dS0),
                            _p(cap_off), _p(cap_pos), _p(cap_out), _p(lam), nthreads or default_threads())
        if rc:
            raise MemoryError("oracle_bwd")
        return dict(dq=dq, dk=dk_, dv=dv_, dg=dg, dbeta=db, dS0=dS0, lam=lam)
