"""ctypes marshalling for ``include/harts.h`` (same names, same arguments).

Host arrays are numpy; device buffers are torch tensors passed by data
pointer, with the current torch stream as the HIP stream.  Every entry point
checks the shapes it can see and raises :class:`HartsError` with the
library's message on a negative return code.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_harts.so")

DTYPE_BF16 = 0
DTYPE_FP32 = 1

if not os.path.exists(_SO):
    raise ImportError("HIP library %s is missing: build it with chunkwise_linear_attention_gated_amd.build.build()"
                      % _SO)
# PyTorch ships its own HIP runtime under the same soname.  Load it first so the
# library binds to that runtime: device pointers and streams handed over from
# torch are only valid inside the runtime instance that created them.
try:
    import torch  # noqa: F401
except ImportError:  # host-only use (planner) without torch
    pass
_L = ctypes.CDLL(_SO)
library = _SO

P = ctypes.c_void_p
I32, I64 = ctypes.c_int32, ctypes.c_int64


class PlanInfo(ctypes.Structure):
    _fields_ = [("S", I64), ("C", I64), ("chunk_B", I32), ("n_rounds", I32), ("min_calls", I32),
                ("n_sequences", I32), ("n_slots", I32), ("n_boundaries", I32), ("replay_total", I64),
                ("n_chunks", I64), ("n_vrows", I64)]


class SeqView(ctypes.Structure):
    _fields_ = [("round", I32), ("init_slot", I32), ("start", I64), ("row_begin", I64), ("row_end", I64),
                ("replay_off", I64), ("n_replay", I32), ("n_emits", I32), ("emit_off", I64)]


class KdaIO(ctypes.Structure):
    _fields_ = [("q", P), ("k", P), ("v", P), ("g", P), ("beta", P), ("o", P), ("states", P),
                ("init_states", P), ("final_states", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t),
                ("keep", I32)]


class KdaGrad(ctypes.Structure):
    _fields_ = [("dO", P), ("dq", P), ("dk", P), ("dv", P), ("dg", P), ("dbeta", P), ("dstates", P), ("dinit", P)]


class RoundView(ctypes.Structure):
    _fields_ = [("n_seq", I32), ("row_start", P), ("row_end", P), ("abs_start", P), ("replay_off", P),
                ("replay_rows", P), ("init_slot", P), ("emit_off", P), ("emit_chunk", P), ("emit_slot", P)]


class VarlenArgs(ctypes.Structure):
    _fields_ = [("q", P), ("k", P), ("v", P), ("g", P), ("beta", P), ("cu_seqlens", P), ("n_seq", I64),
                ("init_states", P), ("init_mask", P), ("o", P), ("boundary_states", P), ("boundary_offsets", P),
                ("final_states", P), ("H", I32), ("dk", I32), ("dv", I32), ("chunk_B", I32), ("dtype", I32)]


class ProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("launches", I64), ("total_ms", ctypes.c_double), ("units", I64)]


def _sig(name, res, *args):
    f = getattr(_L, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_tree_build = _sig("harts_tree_build", I32, P, P, I64, ctypes.POINTER(P))
_tree_stats = _sig("harts_tree_stats", I32, P, P, P, P, P)
_tree_free = _sig("harts_tree_free", None, P)
_plan_create = _sig("harts_plan_create", I32, P, I32, ctypes.POINTER(P))
_plan_create_varlen = _sig("harts_plan_create_varlen", I32, P, I64, I32, P, I32, ctypes.POINTER(P))
_plan_info = _sig("harts_plan_info", I32, P, ctypes.POINTER(PlanInfo))
_plan_maps = _sig("harts_plan_maps", I32, P, P, P, P)
_plan_sequences = _sig("harts_plan_sequences", I32, P, P)
_plan_replay_rows = _sig("harts_plan_replay_rows", I32, P, P)
_plan_emits = _sig("harts_plan_emits", I32, P, P, P)
_plan_boundary_offsets = _sig("harts_plan_boundary_offsets", I32, P, P)
_plan_round = _sig("harts_plan_round", I32, P, I32, ctypes.POINTER(RoundView))
_plan_free = _sig("harts_plan_free", None, P)
_plan_upload = _sig("harts_plan_upload", I32, P, I32, I32, I32, I32, P, ctypes.POINTER(P))
_ws_size = _sig("harts_kda_workspace_size", I32, P, I32, ctypes.POINTER(ctypes.c_size_t))
_dev_free = _sig("harts_dev_plan_free", None, P)
_kda_fwd = _sig("harts_kda_fwd", I32, P, ctypes.POINTER(KdaIO), P)
_kda_bwd = _sig("harts_kda_bwd", I32, P, ctypes.POINTER(KdaIO), ctypes.POINTER(KdaGrad), P)
_kda_fwd_varlen = _sig("harts_kda_fwd_varlen", I32, ctypes.POINTER(VarlenArgs), P)
_lp_ws = _sig("harts_logprob_workspace_size", ctypes.c_size_t, I64)
_lp_ws2 = _sig("harts_logprob_workspace", ctypes.c_size_t, I64, I64)
_lp = _sig("harts_logprob_gather", I32, P, I64, I64, I32, P, P, I64, P, P, P, P, ctypes.c_size_t, P)
_lp_na = _sig("harts_logprob_gather_noalloc", I32, P, I64, I64, I32, P, P, I64, P, P, P)
_lpb = _sig("harts_logprob_backward", I32, P, I64, I64, I32, P, P, P, P, P, I64, P, P)
_lp_rows = _sig("harts_logprob_rows", I32, P, I64, I64, P, P)
_lp_check = _sig("harts_logprob_check_map", I32, P, P, I64, I64, I64)
_conv_tables = _sig("harts_conv_tables", I32, P, P, I64, I64, I32, P, P, P)
_conv_ws = _sig("harts_conv_workspace_size", ctypes.c_size_t, I64, I32, I32)
_conv_fwd = _sig("harts_conv_fwd", I32, P, P, P, I64, I32, I32, I32, P, P)
_attn_build = _sig("harts_attn_tables_build", I32, P, P, I64, I64, ctypes.POINTER(P))
_attn_info = _sig("harts_attn_info", I32, P, P)
_attn_copy = _sig("harts_attn_tables_copy", I32, P, P, P, P, P, P)
_attn_free = _sig("harts_attn_tables_free", None, P)
_attn_ws = _sig("harts_attn_workspace_size", ctypes.c_size_t, I64, I32)
_attn_fwd = _sig("harts_attn_fwd", I32, P, P, P, P, I64, P, I64, I32, I32, I32, ctypes.c_float, P, P, P)
_attn_bwd = _sig("harts_attn_bwd", I32, P, P, P, P, P, P, P, I64, P, P, I64, P, I64, I32, I32, I32, ctypes.c_float,
                 P, P, P, P, ctypes.c_size_t, P)
_moe_ws = _sig("harts_moe_workspace_size", ctypes.c_size_t, I64, I32)
_moe_stats = _sig("harts_moe_stats", I32, P, P, P, I64, I32, I32, I64, P, P, P, P, P, P, ctypes.c_size_t, P)
_moe_grad = _sig("harts_moe_grad", I32, P, P, P, I64, I32, I32, I64, ctypes.c_float, ctypes.c_float, P, P)
_moe_bias = _sig("harts_moe_bias_update", I32, P, I32, ctypes.c_float, P, P)
_conv_bwd = _sig("harts_conv_bwd", I32, P, P, P, P, P, P, I64, I32, I32, I32, P, P, P, ctypes.c_size_t, P)
_prof_enable = _sig("harts_profile_enable", I32, I32)
_prof_collect = _sig("harts_profile_collect", I32, P, I32, P)
_last_error = _sig("harts_last_error", ctypes.c_char_p)
_version = _sig("harts_version", ctypes.c_char_p)


class HartsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("harts error %d: %s" % (code, msg))
        self.code = code


def _check(rc: int):
    if rc != 0:
        raise HartsError(rc, _last_error().decode())


def version() -> str:
    return _version().decode()


def _np(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(0)


class _PlanBase:
    _h = None

    @property
    def info(self) -> PlanInfo:
        inf = PlanInfo()
        _check(_plan_info(self._h, ctypes.byref(inf)))
        return inf

    def maps(self):
        inf = self.info
        m = np.empty(inf.S, np.int64)
        q = np.empty(inf.C, np.int32)
        n2r = np.empty(inf.C, np.int64)
        _check(_plan_maps(self._h, m.ctypes.data, q.ctypes.data, n2r.ctypes.data))
        return m, q, n2r

    def sequences(self):
        inf = self.info
        arr = (SeqView * inf.n_sequences)()
        _check(_plan_sequences(self._h, arr))
        return [dict((f, getattr(s, f)) for f, _ in SeqView._fields_) for s in arr]

    def replay_rows(self) -> np.ndarray:
        inf = self.info
        out = np.empty(inf.replay_total, np.int64)
        _check(_plan_replay_rows(self._h, out.ctypes.data if inf.replay_total else None))
        return out

    def emits(self):
        seqs = self.sequences()
        n = sum(s["n_emits"] for s in seqs)
        b = np.empty(n, np.int32)
        t = np.empty(n, np.int32)
        _check(_plan_emits(self._h, b.ctypes.data, t.ctypes.data))
        return b, t

    def round(self, r: int) -> dict:
        """harts_plan_round: the sequences of round r (0-based) as numpy copies of the
        plan-owned arrays."""
        rv = RoundView()
        _check(_plan_round(self._h, r, ctypes.byref(rv)))
        n = rv.n_seq

        def arr(ptr, count, ctype, dtype):
            if count == 0:
                return np.empty(0, dtype)
            return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctype)), (count,)).astype(dtype)

        out = {"n_seq": n}
        for f in ("row_start", "row_end", "abs_start"):
            out[f] = arr(getattr(rv, f), n, I64, np.int64)
        out["init_slot"] = arr(rv.init_slot, n, I32, np.int32)
        out["replay_off"] = arr(rv.replay_off, n + 1, I64, np.int64)
        out["emit_off"] = arr(rv.emit_off, n + 1, I64, np.int64)
        out["replay_rows"] = arr(rv.replay_rows, int(out["replay_off"][-1]), I64, np.int64)
        out["emit_chunk"] = arr(rv.emit_chunk, int(out["emit_off"][-1]), I32, np.int32)
        out["emit_slot"] = arr(rv.emit_slot, int(out["emit_off"][-1]), I32, np.int32)
        return out

    def __del__(self):
        if self._h:
            _plan_free(self._h)
            self._h = None


class TreePlan(_PlanBase):
    """harts_tree_build + harts_plan_create: trajectories -> compact tokens ->
    minimum-call packed rounds."""

    def __init__(self, tokens, offsets, chunk_B: int):
        tokens = _np(tokens, np.int32)
        offsets = _np(offsets, np.int64)
        self._tree = P()
        _check(_tree_build(tokens.ctypes.data, offsets.ctypes.data, len(offsets) - 1, ctypes.byref(self._tree)))
        h = P()
        _check(_plan_create(self._tree, chunk_B, ctypes.byref(h)))
        self._h = h

    def tree_stats(self):
        v = [I64() for _ in range(4)]
        _check(_tree_stats(self._tree, *[ctypes.byref(x) for x in v]))
        return dict(S=v[0].value, C=v[1].value, n_segments=v[2].value, n_forks=v[3].value)

    def __del__(self):
        super().__del__()
        if getattr(self, "_tree", None):
            _tree_free(self._tree)
            self._tree = None


class VarlenPlan(_PlanBase):
    """harts_plan_create_varlen: independent packed sequences in one call."""

    def __init__(self, cu_seqlens, chunk_B: int, has_init=None, emit_boundaries: bool = False):
        cu = _np(cu_seqlens, np.int64)
        hi = None if has_init is None else _np(has_init, np.uint8)
        h = P()
        _check(_plan_create_varlen(cu.ctypes.data, len(cu) - 1, chunk_B, None if hi is None else hi.ctypes.data,
                                   int(bool(emit_boundaries)), ctypes.byref(h)))
        self._h = h
        self._n = len(cu) - 1

    def boundary_offsets(self) -> np.ndarray:
        out = np.empty(self._n + 1, np.int64)
        _check(_plan_boundary_offsets(self._h, out.ctypes.data))
        return out


class DevicePlan:
    """harts_plan_upload: descriptors on the device for (H, dk, dv, dtype)."""

    def __init__(self, plan: _PlanBase, H: int, dk: int, dv: int, dtype: int, stream=None):
        self.plan = plan
        self.H, self.dk, self.dv, self.dtype = H, dk, dv, dtype
        h = P()
        _check(_plan_upload(plan._h, H, dk, dv, dtype, _stream(stream), ctypes.byref(h)))
        self._h = h

    def workspace_size(self, backward) -> int:
        """backward: False/0 forward, True/1 backward, 2 a forward/backward pair with keep."""
        n = ctypes.c_size_t()
        _check(_ws_size(self._h, int(backward), ctypes.byref(n)))
        return n.value

    def __del__(self):
        if getattr(self, "_h", None):
            _dev_free(self._h)
            self._h = None


def _io(q, k, v, g, beta, o, states, init_states, final_states, workspace, keep):
    return KdaIO(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o), _ptr(states), _ptr(init_states),
                 _ptr(final_states), _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
                 int(bool(keep)))


def kda_fwd(dplan: DevicePlan, q, k, v, g, beta, o, states=None, init_states=None, final_states=None,
            workspace=None, stream=None, keep=False):
    """harts_kda_fwd over every round of the plan (keep: also leave the backward's operands
    and chunk-start states in the workspace for kda_bwd(..., keep=True))."""
    io = _io(q, k, v, g, beta, o, states, init_states, final_states, workspace, keep)
    _check(_kda_fwd(dplan._h, ctypes.byref(io), _stream(stream)))


def kda_fwd_varlen(q, k, v, g, beta, cu_seqlens, o, chunk_B: int, init_states=None, init_mask=None,
                   boundary_states=None, final_states=None, stream=None):
    """harts_kda_fwd_varlen: the flat packed call in one function (plans, uploads, allocates its
    workspace, runs and waits).  q, k, g, o [N, H, dk or dv]; beta [N, H]; cu_seqlens host [n_seq + 1].
    Returns the boundary offsets [n_seq + 1] when boundary_states is given, else None."""
    import torch
    cu = _np(cu_seqlens, np.int64)
    n = len(cu) - 1
    if q.dim() != 3 or v.dim() != 3:
        raise HartsError(-1, "q and v must be [N, H, d]")
    N, H, dk = q.shape
    dv = v.shape[2]
    dtype = DTYPE_BF16 if q.dtype == torch.bfloat16 else DTYPE_FP32
    mask = None if init_mask is None else _np(init_mask, np.uint8)
    if mask is not None and len(mask) != n:
        raise HartsError(-1, "init_mask must have n_seq entries")
    offs = np.empty(n + 1, np.int64) if boundary_states is not None else None
    a = VarlenArgs(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), cu.ctypes.data, n, _ptr(init_states),
                   None if mask is None else mask.ctypes.data, _ptr(o), _ptr(boundary_states),
                   None if offs is None else offs.ctypes.data, _ptr(final_states), H, dk, dv, chunk_B, dtype)
    _check(_kda_fwd_varlen(ctypes.byref(a), _stream(stream)))
    return offs


def kda_bwd(dplan: DevicePlan, q, k, v, g, beta, dO, dq, dk, dv, dg, dbeta, states=None, init_states=None,
            dstates=None, dinit=None, workspace=None, stream=None, keep=False):
    """harts_kda_bwd over every round of the plan, in reverse (keep: read what
    kda_fwd(..., keep=True) left in the same workspace instead of recomputing it)."""
    io = _io(q, k, v, g, beta, None, states, init_states, None, workspace, keep)
    gr = KdaGrad(_ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dstates), _ptr(dinit))
    _check(_kda_bwd(dplan._h, ctypes.byref(io), ctypes.byref(gr), _stream(stream)))


def logprob_workspace_size(C: int) -> int:
    return int(_lp_ws(C))


def logprob_workspace(C: int, S: int) -> int:
    """harts_logprob_workspace: workspace bytes for C compact rows and S semantic positions."""
    return int(_lp_ws2(C, S))


def logprob_gather(logits, m, labels, logp, q=None, lse=None, workspace=None, stream=None):
    """harts_logprob_gather: logp[s] = logits[m[s], labels[s]] - logsumexp(logits[m[s]])."""
    import torch
    C, V = logits.shape
    dtype = DTYPE_BF16 if logits.dtype == torch.bfloat16 else DTYPE_FP32
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise HartsError(-1, "logits must be bf16 or fp32")
    S = m.numel()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lp(_ptr(logits), C, V, dtype, _ptr(m), _ptr(labels), S, _ptr(logp), _ptr(q), _ptr(lse),
               _ptr(workspace), ws_bytes, _stream(stream)))


def logprob_gather_noalloc(logits, m, labels, logp, q=None, stream=None):
    """harts_logprob_gather_noalloc: harts_logprob_gather with the library's own per-device scratch
    (no workspace, no allocation; at most HARTS_LOGPROB_NOALLOC_MAX_ROWS rows)."""
    import torch
    C, V = logits.shape
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise HartsError(-1, "logits must be bf16 or fp32")
    dtype = DTYPE_BF16 if logits.dtype == torch.bfloat16 else DTYPE_FP32
    _check(_lp_na(_ptr(logits), C, V, dtype, _ptr(m), _ptr(labels), m.numel(), _ptr(logp), _ptr(q), _stream(stream)))


def logprob_backward(logits, lse, row_off, row_pos, labels, dlogp, dlogits, stream=None):
    """harts_logprob_backward: dlogits[c] = sum over row c's positions of
    dlogp[s] (onehot(labels[s]) - softmax(logits[c]))."""
    import torch
    C, V = logits.shape
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise HartsError(-1, "logits must be bf16 or fp32")
    dtype = DTYPE_BF16 if logits.dtype == torch.bfloat16 else DTYPE_FP32
    _check(_lpb(_ptr(logits), C, V, dtype, _ptr(lse), _ptr(row_off), _ptr(row_pos), _ptr(labels), _ptr(dlogp),
                labels.numel(), _ptr(dlogits), _stream(stream)))


def logprob_check_map(m, labels, C: int, V: int):
    """harts_logprob_check_map (host): raises HartsError (HARTS_ERANGE) naming the first semantic
    position whose row is outside [0, C) or whose label is outside [0, V)."""
    m = np.ascontiguousarray(m, dtype=np.int64)
    lab = None if labels is None else np.ascontiguousarray(labels, dtype=np.int32)
    _check(_lp_check(m.ctypes.data, None if lab is None else lab.ctypes.data, m.shape[0], C, V))


def logprob_rows(m, C: int):
    """harts_logprob_rows (host): CSR offsets [C + 1] and positions [S] of every compact
    row's semantic positions, in increasing order."""
    m = np.ascontiguousarray(m, dtype=np.int64)
    off = np.empty(C + 1, dtype=np.int64)
    pos = np.empty(m.shape[0], dtype=np.int64)
    _check(_lp_rows(m.ctypes.data, m.shape[0], C, off.ctypes.data, pos.ctypes.data))
    return off, pos


def conv_tables(m, traj_offsets, C: int, w: int):
    """harts_conv_tables (host): ancestor table [C, w - 1] (int32) and the gather lists
    (offsets [C + 1], entries 8 t + j) of the tree causal convolution."""
    m = np.ascontiguousarray(m, dtype=np.int64)
    off = np.ascontiguousarray(traj_offsets, dtype=np.int64)
    anc = np.empty((C, w - 1), dtype=np.int32)
    goff = np.empty(C + 1, dtype=np.int64)
    gl = np.empty(max(1, C * (w - 1)), dtype=np.int64)
    _check(_conv_tables(m.ctypes.data, off.ctypes.data, off.shape[0] - 1, C, w, anc.ctypes.data, goff.ctypes.data,
                        gl.ctypes.data))
    return anc, goff, gl  # gl holds goff[-1] entries (at least one slot, so never empty)


def conv_workspace_size(C: int, channels: int, w: int) -> int:
    return int(_conv_ws(C, channels, w))


def _act_dtype(x):
    import torch
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise HartsError(-1, "activations must be bf16 or fp32")
    return DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_FP32


def conv_fwd(x, weight, anc, out, stream=None):
    """harts_conv_fwd: out[t] = sum_j weight[:, j] * x[anc_j(t)] over the compact rows."""
    C, ch = x.shape
    _check(_conv_fwd(_ptr(x), _ptr(weight), _ptr(anc), C, ch, weight.shape[1], _act_dtype(x), _ptr(out),
                     _stream(stream)))


def conv_bwd(x, weight, anc, gather_off, gather, dout, dx=None, dweight=None, workspace=None, stream=None):
    """harts_conv_bwd: dx and dweight of sum_t <dout[t], out[t]>."""
    C, ch = x.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_conv_bwd(_ptr(x), _ptr(weight), _ptr(anc), _ptr(gather_off), _ptr(gather), _ptr(dout), C, ch,
                     weight.shape[1], _act_dtype(x), _ptr(dx), _ptr(dweight), _ptr(workspace), ws_bytes,
                     _stream(stream)))


class AttnInfo(ctypes.Structure):
    _fields_ = [("C", I64), ("n_segments", I64), ("n_qtiles", I64), ("n_ktiles", I64), ("kv_list_len", I64),
                ("q_list_len", I64), ("pairs", I64), ("max_depth", I32)]


def attn_tables(m, traj_offsets, C: int):
    """harts_attn_tables_build + harts_attn_tables_copy (host): the tree-attention tiles and
    row lists as numpy int32 arrays {qtiles [n, 4], kv_list, ktiles [n, 4], q_list, pos [C]}
    plus the table sizes ("info", a dict)."""
    m = np.ascontiguousarray(m, dtype=np.int64)
    off = np.ascontiguousarray(traj_offsets, dtype=np.int64)
    h = P()
    _check(_attn_build(m.ctypes.data, off.ctypes.data, off.shape[0] - 1, C, ctypes.byref(h)))
    try:
        info = AttnInfo()
        _check(_attn_info(h, ctypes.byref(info)))
        out = {
            "qtiles": np.empty((info.n_qtiles, 4), dtype=np.int32),
            "kv_list": np.empty(max(1, info.kv_list_len), dtype=np.int32),
            "ktiles": np.empty((info.n_ktiles, 4), dtype=np.int32),
            "q_list": np.empty(max(1, info.q_list_len), dtype=np.int32),
            "pos": np.empty(max(1, C), dtype=np.int32),
        }
        _check(_attn_copy(h, *(out[k].ctypes.data for k in ("qtiles", "kv_list", "ktiles", "q_list", "pos"))))
    finally:
        _attn_free(h)
    out["pos"] = out["pos"][:C]
    out["info"] = {f: getattr(info, f) for f, _ in AttnInfo._fields_}
    return out


def attn_workspace_size(C: int, H: int) -> int:
    return int(_attn_ws(C, H))


def _bf16(*xs):
    import torch
    for x in xs:
        if x.dtype != torch.bfloat16 or not x.is_contiguous():
            raise HartsError(-1, "attention operands must be contiguous bf16")


def attn_fwd(q, k, v, qtiles, kv_list, scale: float, o, lse, stream=None):
    """harts_attn_fwd: o[t] = softmax over the rows of t's root path of scale <q[t], k[a]>, times v;
    lse[t] its natural-log denominator.  q, k: [C, H, dqk]; v, o: [C, H, dv] bf16."""
    _bf16(q, k, v, o)
    C, H, dqk = q.shape
    _check(_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(qtiles), qtiles.shape[0], _ptr(kv_list), C, H, dqk,
                     v.shape[2], float(scale), _ptr(o), _ptr(lse), _stream(stream)))


def attn_bwd(q, k, v, o, lse, dout, qtiles, kv_list, ktiles, q_list, scale: float, dq, dk, dv, workspace,
             stream=None):
    """harts_attn_bwd: dq, dk, dv of sum_t <dout[t], o[t]>."""
    _bf16(q, k, v, o, dout, dq, dk, dv)
    C, H, dqk = q.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(qtiles), qtiles.shape[0],
                     _ptr(kv_list), _ptr(ktiles), ktiles.shape[0], _ptr(q_list), C, H, dqk, v.shape[2],
                     float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream)))


def moe_workspace_size(C: int, E: int) -> int:
    return int(_moe_ws(C, E))


def moe_stats(logits, q, k: int, S: int, topk, lse, counts, mass, losses, workspace, bias=None, stream=None):
    """harts_moe_stats: q-weighted router statistics of the compact rows (logits fp32 [C, E])."""
    C, E = logits.shape
    _check(_moe_stats(_ptr(logits), _ptr(bias), _ptr(q), C, E, k, S, _ptr(topk), _ptr(lse), _ptr(counts), _ptr(mass),
                      _ptr(losses), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_grad(logits, q, counts, k: int, S: int, z_coef: float, aux_coef: float, dlogits, stream=None):
    """harts_moe_grad: d(z_coef L_z + aux_coef L_aux)/d logits, counts held fixed."""
    C, E = logits.shape
    _check(_moe_grad(_ptr(logits), _ptr(q), _ptr(counts), C, E, k, S, float(z_coef), float(aux_coef), _ptr(dlogits),
                     _stream(stream)))


def moe_bias_update(counts, gamma: float, bias, stream=None):
    """harts_moe_bias_update: bias[e] += gamma sign(mean(counts) - counts[e])."""
    _check(_moe_bias(_ptr(counts), counts.shape[0], float(gamma), _ptr(bias), _stream(stream)))


def profile_enable(on: bool = True):
    """harts_profile_enable: bracket every library kernel with HIP events."""
    _check(_prof_enable(int(bool(on))))


def profile_collect():
    """harts_profile_collect: {kernel name: (launches, total_ms, units)}."""
    n = I32()
    arr = (ProfileEntry * 64)()
    _check(_prof_collect(arr, 64, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms, arr[i].units) for i in range(min(n.value, 64))}
