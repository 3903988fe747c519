"""GPU parity of the multiplicity-weighted router statistics against the float64 oracle:
random rows with every supported expert count, k = 1 and 8, ties, the rollout tree's
compact rows with their multiplicities, repeat runs, and the bias update.

Routing decisions are compared where the oracle's k-th and (k+1)-th scores differ by more
than 1e-6 (p <= 1, fp32 softmax error ~1e-7); a row within that margin (under 1 % of rows)
may move its weight to the other expert, so counts are exact up to those rows' q_c.  lse
within 1e-5, mass and losses within a relative 1e-5 (fp32 sums of positive terms), gradients
within 1e-5 of their largest entry."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import moe as omoe  # noqa: E402


def _run(z, bias, q, k, S):
    C, E = z.shape
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    tz, tq = dev(z, torch.float32), dev(q, torch.int32)
    tb = None if bias is None else dev(bias, torch.float32)
    top = torch.full((C, k), -1, dtype=torch.int32, device="cuda")
    lse = torch.full((C,), float("nan"), device="cuda")
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    mass = torch.full((E,), float("nan"), device="cuda")
    losses = torch.full((2,), float("nan"), device="cuda")
    ws = torch.empty(harts.moe_workspace_size(C, E), dtype=torch.uint8, device="cuda")
    harts.moe_stats(tz, tq, k, S, top, lse, counts, mass, losses, ws, bias=tb)
    dz = torch.full_like(tz, float("nan"))
    harts.moe_grad(tz, tq, counts, k, S, 0.7, 1.9, dz)
    torch.cuda.synchronize()
    return {"top": top.cpu().numpy(), "lse": lse.cpu().numpy(), "counts": counts.cpu().numpy(),
            "mass": mass.cpu().numpy(), "losses": losses.cpu().numpy(), "dz": dz.cpu().numpy()}


def _check(z, bias, q, k, S):
    got = _run(z, bias, q, k, S)
    b = np.zeros(z.shape[1]) if bias is None else bias
    st = omoe.statistics(z.astype(np.float32).astype(np.float64), b, q, k, S)
    p, _, _ = omoe.route(z, b, k)
    srt = -np.sort(-(p + b[None, :]), axis=1)
    margin = (srt[:, k - 1] - srt[:, k]) if k < z.shape[1] else np.full(len(z), np.inf)
    amb = margin <= 1e-6  # the k-th choice is within fp32 rounding of the next one
    assert amb.mean() < 1e-2
    ok = ~amb
    assert np.array_equal(got["top"][ok], st["top"][ok])
    # an ambiguous row may move its q_c from one expert to another
    slack = int(np.asarray(q)[amb].sum())
    assert np.abs(got["counts"].astype(np.int64) - st["counts"]).max() <= slack
    assert got["counts"].sum() == st["counts"].sum()
    assert np.abs(got["lse"] - st["lse"]).max() <= 1e-5
    np.testing.assert_allclose(got["mass"], st["mass"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(got["losses"], [st["L_z"], st["L_aux"]], rtol=1e-5)
    g = omoe.grad(z, b, q, k, S, 0.7, 1.9)
    assert np.abs(got["dz"] - g).max() <= 1e-5 * np.abs(g).max()
    return got


@pytest.mark.parametrize("E", [64, 128, 256])
@pytest.mark.parametrize("k", [1, 8])
def test_moe_random_rows(E, k):
    rng = np.random.default_rng(E + k)
    C = 300
    z = (rng.standard_normal((C, E)) * 1.5).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.01).astype(np.float32)
    q = rng.integers(1, 9, C)
    _check(z, bias, q, k, int(q.sum()))


def test_moe_ties_take_the_lower_expert():
    z = np.zeros((5, 64), np.float32)
    got = _run(z, None, np.ones(5, np.int64), 4, 5)
    assert (got["top"] == np.arange(4)[None, :]).all()
    assert got["counts"][:4].tolist() == [5, 5, 5, 5] and got["counts"][4:].sum() == 0


def test_moe_rollout_tree_rows_and_repeat():
    from synthetic import trees
    t = trees.random_rollout_tree(seed=0)
    hp = harts.TreePlan(t.tokens, t.offsets, 64)
    m = np.asarray(hp.maps()[0], np.int64)
    C = hp.info.C
    q = np.bincount(m, minlength=C)
    rng = np.random.default_rng(3)
    z = (rng.standard_normal((C, 128)) * 2.0).astype(np.float32)
    bias = (rng.standard_normal(128) * 0.01).astype(np.float32)
    got = _check(z, bias, q, 8, len(m))
    again = _run(z, bias, q, 8, len(m))
    for key in got:
        assert np.array_equal(got[key], again[key]), key


def test_moe_bias_update():
    rng = np.random.default_rng(4)
    counts = rng.integers(0, 50, 128).astype(np.int32)
    counts[5] = int(round(counts.mean()))  # may or may not equal the mean exactly
    b0 = (rng.standard_normal(128) * 0.1).astype(np.float32)
    tb = torch.from_numpy(b0.copy()).cuda()
    harts.moe_bias_update(torch.from_numpy(counts).cuda(), 0.001, tb)
    ref = (b0.astype(np.float32) + np.float32(0.001) * np.sign(counts.mean() - counts).astype(np.float32))
    np.testing.assert_array_equal(tb.cpu().numpy(), ref.astype(np.float32))
