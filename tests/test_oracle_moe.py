"""Pins of the multiplicity-weighted MoE statistics oracle: compact rows with weights q_c
against the library's softmax / logsumexp / topk / bincount run on the expanded semantic
rows, the gradient against autograd of the expanded losses, ties, and a hand example of
the bias update."""
import numpy as np
import torch

from oracle import moe


def _case(seed, C=40, E=16, S_extra=60):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((C, E)) * 1.5
    bias = rng.standard_normal(E) * 0.05
    m = np.concatenate([np.arange(C), rng.integers(0, C, S_extra)])  # every row read at least once
    rng.shuffle(m)
    return z, bias, m


def test_weighted_statistics_equal_the_expanded_rows():
    z, bias, m = _case(0)
    k, (C, E), S = 4, z.shape, len(m)
    q = np.bincount(m, minlength=C)
    st = moe.statistics(z, bias, q, k, S)
    Z = torch.from_numpy(z[m])
    p = torch.softmax(Z, dim=1)
    lse = torch.logsumexp(Z, dim=1)
    top = torch.topk(p + torch.from_numpy(bias), k, dim=1).indices
    n = torch.bincount(top.flatten(), minlength=E).numpy()
    P = p.sum(dim=0).numpy()
    assert np.array_equal(st["counts"], n)
    np.testing.assert_allclose(st["mass"], P, rtol=0, atol=1e-12)
    np.testing.assert_allclose(st["L_z"], float((lse ** 2).mean()), rtol=1e-13)
    np.testing.assert_allclose(st["L_aux"], E / (k * S * S) * float((n * P).sum()), rtol=1e-13)
    # routing decisions are the expanded rows' decisions
    assert np.array_equal(st["top"][m], top.numpy())


def test_gradient_equals_autograd_of_the_expanded_losses():
    z, bias, m = _case(1)
    k, (C, E), S = 3, z.shape, len(m)
    q = np.bincount(m, minlength=C)
    zc, ac = 0.7, 1.9
    g = moe.grad(z, bias, q, k, S, zc, ac)
    tz = torch.tensor(z, requires_grad=True)
    Z = tz[torch.from_numpy(m)]
    p = torch.softmax(Z, dim=1)
    lse = torch.logsumexp(Z, dim=1)
    top = torch.topk(p.detach() + torch.from_numpy(bias), k, dim=1).indices
    n = torch.bincount(top.flatten(), minlength=E).double()
    loss = zc * (lse ** 2).mean() + ac * E / (k * S * S) * (n * p.sum(dim=0)).sum()
    loss.backward()
    np.testing.assert_allclose(g, tz.grad.numpy(), rtol=0, atol=1e-14)


def test_ties_take_the_lower_expert():
    z = np.zeros((2, 8))
    _, _, top = moe.route(z, np.zeros(8), 3)
    assert top.tolist() == [[0, 1, 2], [0, 1, 2]]
    _, _, top = moe.route(z, np.array([0, 0, 0, 0, 1e-3, 0, 0, 1e-3]), 3)
    assert top.tolist()[0] == [4, 7, 0]


def test_bias_update_by_hand():
    b = moe.bias_update(np.array([0.0, 0.1, -0.1, 0.0]), np.array([3, 5, 1, 3]), 0.01)
    # mean count 3: above -> down, below -> up, equal -> unchanged
    np.testing.assert_allclose(b, [0.0, 0.09, -0.09, 0.0], rtol=0, atol=1e-15)
