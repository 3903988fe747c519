"""GPU parity of the fused compact-row log-softmax + gather and the occurrence
counts against the float64 oracle (small shapes, both dtypes, ragged V)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import logprob as olp  # noqa: E402
from synthetic import tensors  # noqa: E402


def _run(C, V, dtype, seed):
    w = tensors.logprob_map(C, V, seed=seed)
    x = tensors.logits_torch(C, V, seed=seed, device="cuda", dtype=dtype)
    m = torch.from_numpy(w.m).cuda()
    lab = torch.from_numpy(w.labels).cuda()
    logp = torch.empty(len(w.m), dtype=torch.float32, device="cuda")
    q = torch.empty(C, dtype=torch.int32, device="cuda")
    ws = torch.empty(harts.logprob_workspace_size(C), dtype=torch.uint8, device="cuda")
    harts.logprob_gather(x, m, lab, logp, q=q, workspace=ws)
    torch.cuda.synchronize()
    ref = olp.logprob(x.float().cpu().numpy().astype(np.float64), w.m, w.labels)
    return w, logp.cpu().numpy(), q.cpu().numpy(), ref


@pytest.mark.parametrize("C,V", [(64, 4096), (33, 1000), (7, 131), (1, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_logprob_small(C, V, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w, lp, q, ref = _run(C, V, dt, seed=C + V)
    assert np.abs(lp - ref).max() <= 1e-3
    assert np.array_equal(q, olp.counts(w.m, C))


def test_logprob_constant_rows():
    C, V = 5, 4096
    x = torch.full((C, V), 3.0, dtype=torch.bfloat16, device="cuda")
    m = torch.arange(C, dtype=torch.int64, device="cuda")
    lab = torch.zeros(C, dtype=torch.int32, device="cuda")
    lp = torch.empty(C, dtype=torch.float32, device="cuda")
    lse = torch.empty(C, dtype=torch.float32, device="cuda")
    harts.logprob_gather(x, m, lab, lp, lse=lse)
    torch.cuda.synchronize()
    assert np.abs(lp.cpu().numpy() + np.log(V)).max() < 1e-5


def test_logprob_empty_semantic_set():
    C, V = 4, 64
    x = torch.randn(C, V, device="cuda")
    m = torch.empty(0, dtype=torch.int64, device="cuda")
    lab = torch.empty(0, dtype=torch.int32, device="cuda")
    lp = torch.empty(0, dtype=torch.float32, device="cuda")
    q = torch.full((C,), 7, dtype=torch.int32, device="cuda")
    ws = torch.empty(harts.logprob_workspace_size(C), dtype=torch.uint8, device="cuda")
    harts.logprob_gather(x, m, lab, lp, q=q, workspace=ws)
    torch.cuda.synchronize()
    assert (q.cpu().numpy() == 0).all()


# ---------------------------------------------------------------------------------------------
# backward (equation 19): dlogits against the float64 expanded per-position definition


def _bwd(x, m, lab, g, C):
    """Forward for lse, then the backward; returns dlogits as float64 numpy."""
    S = len(m)
    md = torch.from_numpy(np.asarray(m, np.int64)).cuda()
    ld = torch.from_numpy(np.asarray(lab, np.int32)).cuda()
    lp = torch.empty(S, dtype=torch.float32, device="cuda")
    lse = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    harts.logprob_gather(x, md, ld, lp, lse=lse)
    off, pos = harts.logprob_rows(m, C)
    dx = torch.full_like(x, float("nan"))
    harts.logprob_backward(x, lse, torch.from_numpy(off).cuda(), torch.from_numpy(pos).cuda(), ld,
                           torch.from_numpy(np.asarray(g, np.float32)).cuda(), dx)
    torch.cuda.synchronize()
    return dx.double().cpu().numpy()


def _check_bwd(got, ref, m, g, C, dtype):
    assert not np.isnan(got).any(), "unwritten entries"
    scale = np.zeros(C)
    np.add.at(scale, np.asarray(m, np.int64), np.abs(np.asarray(g, np.float64)))
    rel = 2.0 ** -8 if dtype == torch.bfloat16 else 1e-5
    bound = rel * np.abs(ref) + 1e-6 * (scale[:, None] + 1e-30)
    assert (np.abs(got - ref) <= bound).all(), np.abs(got - ref).max()


@pytest.mark.parametrize("C,V", [(64, 4096), (33, 1000), (7, 131), (1, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_logprob_backward_small(C, V, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w = tensors.logprob_map(C, V, seed=C + V)
    x = tensors.logits_torch(C, V, seed=C + V, device="cuda", dtype=dt)
    g = np.random.default_rng(C).standard_normal(len(w.m))
    got = _bwd(x, w.m, w.labels, g, C)
    ref = olp.logprob_backward(x.double().cpu().numpy(), w.m, w.labels, g.astype(np.float32))
    _check_bwd(got, ref, w.m, g, C, dt)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_logprob_backward_repeated_labels_and_unread_rows(dtype):
    """Several positions of one row with the same label (their weights add), rows no position
    reads (gradient zero), a row read by many positions, and V not a multiple of 16 bytes."""
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    C, V = 9, 333
    rng = np.random.default_rng(2)
    m = np.array([0, 0, 0, 2, 2, 5] + [7] * 80)
    lab = np.array([4, 4, 9, 0, 0, 332] + list(rng.integers(0, 6, size=80)))
    g = rng.standard_normal(len(m))
    x = (torch.randn(C, V, generator=torch.Generator().manual_seed(3)) * 3).to(dt).cuda()
    got = _bwd(x, m, lab, g, C)
    ref = olp.logprob_backward(x.double().cpu().numpy(), m, lab, g.astype(np.float32))
    _check_bwd(got, ref, m, g, C, dt)
    assert (got[[1, 3, 4, 6, 8]] == 0).all() and not np.signbit(got[[1, 3, 4, 6, 8]]).any()


def test_logprob_backward_no_positions_and_repeat_runs_identical():
    C, V = 6, 4096
    x = torch.randn(C, V, device="cuda").to(torch.bfloat16)
    assert (_bwd(x, np.zeros(0, np.int64), np.zeros(0, np.int32), np.zeros(0), C) == 0).all()
    w = tensors.logprob_map(C, V, seed=4)
    g = np.random.default_rng(4).standard_normal(len(w.m))
    a = _bwd(x, w.m, w.labels, g, C)
    b = _bwd(x, w.m, w.labels, g, C)
    assert np.array_equal(a, b)


def test_gather_positions_out_of_range_get_nan_and_are_not_counted():
    C, V = 9, 300
    x = torch.randn((C, V), device="cuda").to(torch.bfloat16)
    m = np.array([0, 3, 9, -1, 8, 3, 2], np.int64)
    lab = np.array([1, 299, 4, 4, 300, -5, 7], np.int32)
    logp = torch.zeros(len(m), device="cuda")
    q = torch.full((C,), -7, dtype=torch.int32, device="cuda")
    harts.logprob_gather(x, torch.from_numpy(m).cuda(), torch.from_numpy(lab).cuda(), logp, q=q,
                         workspace=torch.empty(harts.logprob_workspace_size(C), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    got = logp.cpu().numpy()
    ok = (m >= 0) & (m < C) & (lab >= 0) & (lab < V)
    assert np.isnan(got[~ok]).all() and np.isfinite(got[ok]).all()
    xr = x.double().cpu().numpy()
    ref = olp.logprob(xr, m[ok], lab[ok])
    assert np.abs(got[ok] - ref).max() <= 1e-3
    assert np.array_equal(q.cpu().numpy(), np.bincount(m[ok], minlength=C).astype(np.int32))
