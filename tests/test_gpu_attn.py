"""GPU parity of tree softmax attention (forward o and lse, backward dq, dk, dv) against
the float64 oracle: small trees, forests and chains with ragged and exact tiles, every
supported head-dim pair, and sampled rows of the 64-leaf rollout tree at the benchmark's
head count and dims.

Tolerances, from the arithmetic: inputs are bf16 and exact on both sides; the kernels
round the softmax probabilities P and dS to bf16 for the value-side products (relative
2^-9 each), accumulate in fp32 and store bf16 (2^-9).  So |o - ref| <= 3 * 2^-9 max|v|
(checked at 2^-7 max|v|), lse (fp32 throughout) within 1e-3, and each gradient within
2^-6 of its largest entry plus 1e-4 (norm-wise within 2^-7)."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import attention as oatt  # noqa: E402
from synthetic import trees  # noqa: E402


def _maps(t):
    hp = harts.TreePlan(t.tokens, t.offsets, 64)
    return np.asarray(hp.maps()[0], np.int64), np.asarray(t.offsets, np.int64), hp.info.C


class _Run:
    """Device tables + one forward and backward of the library on seeded bf16 inputs."""

    def __init__(self, m, off, C, H, dqk, dv, seed, gen_on_gpu=False, inputs=None):
        tb = harts.attn_tables(m, off, C)
        self.tb = tb
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.qt, self.kv, self.kt, self.ql = dev(tb["qtiles"]), dev(tb["kv_list"]), dev(tb["ktiles"]), dev(tb["q_list"])
        if inputs is not None:  # float arrays [C, H, d]: q, k, v, dout
            self.q, self.k, self.v, self.do = (torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).cuda()
                                               for a in inputs)
        elif gen_on_gpu:
            g = torch.Generator(device="cuda").manual_seed(seed)
            mk = lambda d: torch.randn((C, H, d), generator=g, device="cuda").to(torch.bfloat16)
            self.q, self.k, self.v, self.do = mk(dqk), mk(dqk), mk(dv), mk(dv)
        else:
            rng = np.random.default_rng(seed)
            mk = lambda d: torch.from_numpy(rng.standard_normal((C, H, d)).astype(np.float32)).to(torch.bfloat16).cuda()
            self.q, self.k, self.v, self.do = mk(dqk), mk(dqk), mk(dv), mk(dv)
        self.scale = 1.0 / math.sqrt(dqk)
        self.o = torch.full((C, H, dv), float("nan"), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.full((C, H), float("nan"), device="cuda")
        harts.attn_fwd(self.q, self.k, self.v, self.qt, self.kv, self.scale, self.o, self.lse)
        self.dq = torch.full_like(self.q, float("nan"))
        self.dk = torch.full_like(self.k, float("nan"))
        self.dv = torch.full_like(self.v, float("nan"))
        ws = torch.empty(harts.attn_workspace_size(C, H), dtype=torch.uint8, device="cuda")
        harts.attn_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.qt, self.kv, self.kt, self.ql,
                       self.scale, self.dq, self.dk, self.dv, ws)
        torch.cuda.synchronize()


def _np(x):
    return x.double().cpu().numpy()


def _close(got, ref, tol, what, atol=1e-4):
    # atol: where every ds term is zero in exact arithmetic (a one-key path), the kernel's ds is
    # the difference of two fp32 sums of <v, dout> taken in different orders
    assert not np.isnan(got).any(), what
    err = np.abs(got - ref).max()
    assert err <= tol * np.abs(ref).max() + atol, (what, err, np.abs(ref).max())


def _check_full(r, m, off):
    q, k, v, do = (_np(x) for x in (r.q, r.k, r.v, r.do))
    o, lse = oatt.attention_forward(q, k, v, m, off, r.scale)
    dq, dk, dv = oatt.attention_backward(q, k, v, do, m, off, r.scale)
    got_o = _np(r.o)
    assert not np.isnan(got_o).any()
    assert np.abs(got_o - o).max() <= 2.0 ** -7 * np.abs(v).max()
    assert np.abs(_np(r.lse) - lse).max() <= 1e-3
    for got, ref, name in ((r.dq, dq, "dq"), (r.dk, dk, "dk"), (r.dv, dv, "dv")):
        g = _np(got)
        _close(g, ref, 2.0 ** -6, name)
        assert np.linalg.norm(g - ref) <= 2.0 ** -7 * np.linalg.norm(ref), name


_DIMS = [(192, 128), (128, 128), (64, 64)]


@pytest.mark.parametrize("dims", _DIMS)
def test_attn_small_trees(dims):
    dqk, dv = dims
    cases = [trees.tiny_tree("G"),
             trees.random_small_tree(np.random.default_rng(3), max_segments=9, max_len=150),
             trees.random_small_tree(np.random.default_rng(4), max_segments=8, max_len=90, forest=True)]
    for i, t in enumerate(cases):
        m, off, C = _maps(t)
        print(f"attn small tree {i}: C={C} dims={dims}", flush=True)
        _check_full(_Run(m, off, C, 2, dqk, dv, seed=10 + i), m, off)


def test_attn_chains_and_ragged_tiles():
    # one chain spanning several tiles, and forests of sequences around the 64-row operand tiles
    # and the 128-row query and key tiles
    for i, lens in enumerate([[300], [1, 63, 64, 65, 130], [127, 128, 129, 260]]):
        t = trees.forest_of_sequences(lens, seed=i)
        m, off, C = _maps(t)
        print(f"attn chains {lens}: C={C}", flush=True)
        _check_full(_Run(m, off, C, 3, 192, 128, seed=20 + i), m, off)


@pytest.mark.parametrize("trend", [1.0, -1.0])
def test_attn_scores_rising_or_falling_along_the_path(trend):
    """Scores whose maximum rises by about 10 (base 2) from one 64-key tile to the next move the
    forward's softmax reference on every tile; falling scores leave it at the first tile and add
    probabilities far below 1 from the later ones.  One chain of 520 rows (nine 64-key tiles)."""
    dqk, dv, H = 192, 128, 2
    t = trees.forest_of_sequences([520], seed=0)
    m, off, C = _maps(t)
    rng = np.random.default_rng(17)
    u = rng.standard_normal(dqk)
    u *= np.sqrt(dqk) / np.linalg.norm(u)
    pos = np.empty(C)
    pos[m] = np.arange(len(m))  # the position of each compact row on the chain
    b = (pos / 64.0) if trend > 0 else (pos.max() - pos) / 64.0
    q = 0.5 * u[None, None, :] + 0.3 * rng.standard_normal((C, H, dqk))
    k = b[:, None, None] * u[None, None, :] + 0.3 * rng.standard_normal((C, H, dqk))
    v = rng.standard_normal((C, H, dv))
    do = rng.standard_normal((C, H, dv))
    r = _Run(m, off, C, H, dqk, dv, seed=0, inputs=(q, k, v, do))
    qq, kk, vv, dd = (_np(x) for x in (r.q, r.k, r.v, r.do))
    o, lse = oatt.attention_forward(qq, kk, vv, m, off, r.scale)
    dq, dk, dvv = oatt.attention_backward(qq, kk, vv, dd, m, off, r.scale)
    got_o = _np(r.o)
    assert np.isfinite(got_o).all()
    assert np.abs(got_o - o).max() <= 2.0 ** -7 * np.abs(vv).max()
    assert np.abs(_np(r.lse) - lse).max() <= 1e-3
    for got, ref, name in ((r.dk, dk, "dk"), (r.dv, dvv, "dv")):
        g = _np(got)
        _close(g, ref, 2.0 ** -6, name)
        assert np.linalg.norm(g - ref) <= 2.0 ** -7 * np.linalg.norm(ref), name
    # dq = scale sum_j ds_j k_j with sum_j ds_j = 0: the keys' large common part (b_j u) cancels
    # in exact arithmetic, but not once ds_j = p_j (dp_j - delta) is rounded to bf16 for the matrix
    # cores (relative 2^-9) with delta taken from the bf16 output.  Per row and head the error is
    # held to 2^-7 scale sum_j (|ds_j| + p_j sum_e |dout_e o_e|) max|k_j|, four times those roundings.
    g = _np(r.dq)
    assert np.isfinite(g).all()
    P = oatt.paths(m, off, C)
    kmax = np.abs(kk).max(axis=2)  # [C, H]
    for t_ in range(C):
        for h in range(H):
            _, _, p_, ds = oatt.row_terms(qq, kk, vv, dd, P[t_], t_, h, r.scale)
            dabs = np.abs(dd[t_, h] * o[t_, h]).sum()
            bound = 2.0 ** -7 * r.scale * ((np.abs(ds) + p_ * dabs) @ kmax[P[t_], h]) + 1e-4
            err = np.abs(g[t_, h] - dq[t_, h]).max()
            assert err <= bound, ("dq", t_, h, err, bound)


def test_attn_single_row():
    m, off = np.array([0], np.int64), np.array([0, 1], np.int64)
    r = _Run(m, off, 1, 1, 64, 64, seed=5)
    np.testing.assert_allclose(_np(r.o), _np(r.v), rtol=0, atol=0)  # softmax over one key
    # ds = p (dp - delta) with p = 1: zero up to the two fp32 summation orders of <v, dout>
    assert np.abs(_np(r.dq)).max() <= 1e-4 and np.abs(_np(r.dk)).max() <= 1e-4
    np.testing.assert_allclose(_np(r.dv), _np(r.do), rtol=0, atol=0)


def test_attn_repeat_runs_identical():
    t = trees.random_small_tree(np.random.default_rng(8), max_segments=8, max_len=300)
    m, off, C = _maps(t)
    a, b = _Run(m, off, C, 2, 192, 128, seed=1), _Run(m, off, C, 2, 192, 128, seed=1)
    for x, y in ((a.o, b.o), (a.lse, b.lse), (a.dq, b.dq), (a.dk, b.dk), (a.dv, b.dv)):
        assert torch.equal(x, y)


def test_attn_rollout_tree_sampled():
    """The benchmark's rollout tree (64 leaves), 16 heads, dims (192, 128): sampled query rows
    (o, lse, dq) and sampled key rows with at most a few hundred readers (dk, dv)."""
    t = trees.random_rollout_tree(seed=0)
    m, off, C = _maps(t)
    H = 16
    print(f"attn rollout tree: C={C}", flush=True)
    r = _Run(m, off, C, H, 192, 128, seed=7, gen_on_gpu=True)
    parent = oatt.parent_rows(m, off, C)
    rng = np.random.default_rng(0)
    depth = r.tb["pos"].astype(np.int64)

    def terms(t_, h, path):
        idx = torch.from_numpy(path).cuda()
        sub = lambda x: x.index_select(0, idx)[:, h:h + 1].double().cpu().numpy()
        kk, vv = sub(r.k), sub(r.v)
        qq = r.q[t_:t_ + 1, h:h + 1].double().cpu().numpy()
        gg = r.do[t_:t_ + 1, h:h + 1].double().cpu().numpy()
        # local arrays: the query is row 0 of qq/gg, the path is rows 0..L-1 of kk/vv
        o, lse, p, ds = oatt.row_terms(qq, kk, vv, gg, np.arange(len(path)), 0, 0, r.scale)
        return o, lse, p, ds, kk[:, 0], qq[0, 0], gg[0, 0]

    rows = list(rng.choice(C, 24, replace=False)) + [int(np.argmax(depth)), 0]
    for t_ in rows:
        h = int(rng.integers(0, H))
        path = oatt.path_of(parent, int(t_))
        o, lse, p, ds, kk, _, _ = terms(int(t_), h, path)
        got = r.o[t_, h].double().cpu().numpy()
        assert np.abs(got - o).max() <= 2.0 ** -7 * np.abs(_np(r.v.index_select(0, torch.from_numpy(path).cuda())[:, h])).max()
        assert abs(float(r.lse[t_, h]) - lse) <= 1e-3
        dq = r.scale * ds @ kk
        _close(r.dq[t_, h].double().cpu().numpy(), dq, 2.0 ** -6, f"dq row {t_}")

    # key rows with a bounded set of readers (the row and everything below it)
    kids = [[] for _ in range(C)]
    for c in range(C):
        if parent[c] >= 0:
            kids[parent[c]].append(c)
    size = np.ones(C, np.int64)
    for c in np.argsort(-depth, kind="stable"):
        if parent[c] >= 0:
            size[parent[c]] += size[c]
    cand = np.flatnonzero((size >= 2) & (size <= 400))
    keys = list(rng.choice(cand, 8, replace=False)) + [int(np.flatnonzero(size == size[size <= 400].max())[0])]
    for a in keys:
        h = int(rng.integers(0, H))
        readers, stack = [], [int(a)]
        while stack:
            x = stack.pop()
            readers.append(x)
            stack.extend(kids[x])
        dk = np.zeros(192)
        dv = np.zeros(128)
        for t_ in readers:
            path = oatt.path_of(parent, t_)
            _, _, p, ds, _, qv, gv = terms(t_, h, path)
            j = int(np.flatnonzero(path == a)[0])
            dk += r.scale * ds[j] * qv
            dv += p[j] * gv
        _close(r.dk[a, h].double().cpu().numpy(), dk, 2.0 ** -6, f"dk row {a}")
        _close(r.dv[a, h].double().cpu().numpy(), dv, 2.0 ** -6, f"dv row {a}")
