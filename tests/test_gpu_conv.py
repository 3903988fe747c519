"""GPU parity of the tree causal convolution (forward, dx, dweight) against the
float64 per-trajectory oracle: small trees and forests, every supported window
width, both dtypes, and the 64-leaf rollout tree's compact rows."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import conv as oconv  # noqa: E402
from synthetic import trees  # noqa: E402


def _maps(t):
    hp = harts.TreePlan(t.tokens, t.offsets, 64)
    m = hp.maps()[0]
    return np.asarray(m, np.int64), np.asarray(t.offsets, np.int64), hp.info.C


def _run(m, off, C, ch, w, dt, seed):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((C, ch)).astype(np.float32)).to(dt).cuda()
    dout = torch.from_numpy(rng.standard_normal((C, ch)).astype(np.float32)).to(dt).cuda()
    wt = torch.from_numpy(rng.standard_normal((ch, w)).astype(np.float32) / w).cuda()
    anc, goff, gl = harts.conv_tables(m, off, C, w)
    ancd = torch.from_numpy(anc).cuda()
    out = torch.full_like(x, float("nan"))
    harts.conv_fwd(x, wt, ancd, out)
    dx = torch.full_like(x, float("nan"))
    dw = torch.full((ch, w), float("nan"), device="cuda")
    ws = torch.empty(harts.conv_workspace_size(C, ch, w), dtype=torch.uint8, device="cuda")
    harts.conv_bwd(x, wt, ancd, torch.from_numpy(goff).cuda(), torch.from_numpy(gl).cuda(), dout, dx=dx, dweight=dw,
                   workspace=ws)
    torch.cuda.synchronize()
    return (x.double().cpu().numpy(), wt.double().cpu().numpy(), dout.double().cpu().numpy(),
            out.double().cpu().numpy(), dx.double().cpu().numpy(), dw.double().cpu().numpy())


def _close(got, ref, scale, dt):
    assert not np.isnan(got).any()
    rel = 2.0 ** -8 if dt == torch.bfloat16 else 1e-5
    assert (np.abs(got - ref) <= rel * np.abs(ref) + 1e-5 * scale).all(), np.abs(got - ref).max()


@pytest.mark.parametrize("w", [2, 3, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_conv_small_trees(w, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for seed, t in [(1, trees.figure2_tree()),
                    (2, trees.random_small_tree(np.random.default_rng(5), max_segments=9, max_len=40, forest=True)),
                    (3, trees.forest_of_sequences([1, 2, 7, 30]))]:
        m, off, C = _maps(t)
        x, wt, dout, out, dx, dw = _run(m, off, C, 16, w, dt, seed)
        ref = oconv.conv_forward(x, wt, m, off)
        rdx, rdw = oconv.conv_backward(x, wt, m, off, dout)
        _close(out, ref, np.abs(x).max() * np.abs(wt).sum(axis=1).max(), dt)
        _close(dx, rdx, np.abs(dout).max() * np.abs(wt).sum(axis=1).max(), dt)
        _close(dw, rdw, np.abs(dout).max() * np.abs(x).max() * C, torch.float32)


def test_conv_rollout_tree_rows():
    """The 64-leaf rollout tree (73k compact rows) at 64 channels, w = 4: every row's output and
    input gradient and the weight gradient."""
    t = trees.random_rollout_tree(seed=0)
    m, off, C = _maps(t)
    x, wt, dout, out, dx, dw = _run(m, off, C, 64, 4, torch.bfloat16, 11)
    anc, goff, gl = harts.conv_tables(m, off, C, 4)
    # expected rows through the oracle's own trajectory walk on a sample of rows
    rows = np.sort(np.random.default_rng(3).choice(C, size=300, replace=False))
    first = oconv._first_positions(m, off)
    for r in rows:
        tr, p = first[int(r)]
        seq = m[off[tr]:off[tr + 1]]
        want = sum(wt[:, j] * x[seq[p - j]] for j in range(4) if p - j >= 0)
        assert (np.abs(out[r] - want) <= 2.0 ** -8 * np.abs(want) + 1e-4).all()
    rdx, rdw = oconv.conv_backward(x, wt, m, off, dout)
    assert (np.abs(dx - rdx) <= 2.0 ** -8 * np.abs(rdx) + 1e-4).all()
    assert (np.abs(dw - rdw) <= 1e-5 * np.abs(rdw) + 1e-3).all()


def test_conv_repeat_runs_identical():
    t = trees.random_small_tree(np.random.default_rng(8), max_segments=8, max_len=300)
    m, off, C = _maps(t)
    a = _run(m, off, C, 32, 4, torch.bfloat16, 4)
    b = _run(m, off, C, 32, 4, torch.bfloat16, 4)
    for u, v in zip(a[3:], b[3:]):
        assert np.array_equal(u, v)
