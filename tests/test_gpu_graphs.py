"""HIP-graph capture of the paths beside the gated-delta calls: the tree attention (forward and
backward), the tree convolution (forward and both gradients), the log-prob gather (with the
workspace and without), its backward, and the router statistics with their gradient.  Each
call sequence, captured once, replays bit for bit what the eager calls produce, replay after
replay, with eager work between the replays; none of these paths records a memset or an
allocation (counters and partial sums are cleared by kernels)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from synthetic import trees  # noqa: E402


def _maps(t):
    hp = harts.TreePlan(t.tokens, t.offsets, 64)
    return np.asarray(hp.maps()[0], np.int64), np.asarray(t.offsets, np.int64), hp.info.C


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _replay_matches_eager(step, outs):
    """outs: the output tensors step() writes (fixed addresses, so the graph writes them too)."""
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()  # warm-up on a side stream, as capture requires
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.fill_(-7 if not o.is_floating_point() else float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs)):
            assert torch.equal(a, b), ("replay", r, "output", i)
        step()  # eager work between replays
        torch.cuda.synchronize()


def test_attention_graph_replay():
    t = trees.random_small_tree(np.random.default_rng(12), max_segments=8, max_len=300)
    m, off, C = _maps(t)
    H, dqk, dv = 2, 192, 128
    tb = harts.attn_tables(m, off, C)
    qt, kv, kt, ql = (_dev(tb[k]) for k in ("qtiles", "kv_list", "ktiles", "q_list"))
    gen = torch.Generator(device="cuda").manual_seed(3)
    mk = lambda d: torch.randn((C, H, d), generator=gen, device="cuda").to(torch.bfloat16)  # noqa: E731
    q, k, v, do = mk(dqk), mk(dqk), mk(dv), mk(dv)
    o, lse = torch.empty_like(v), torch.empty((C, H), device="cuda")
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(harts.attn_workspace_size(C, H), dtype=torch.uint8, device="cuda")
    scale = dqk ** -0.5
    print(f"attention graph: C={C}", flush=True)

    def step():
        harts.attn_fwd(q, k, v, qt, kv, scale, o, lse)
        harts.attn_bwd(q, k, v, o, lse, do, qt, kv, kt, ql, scale, dq, dk, dvv, ws)

    _replay_matches_eager(step, [o, lse, dq, dk, dvv])


def test_conv_graph_replay():
    t = trees.random_small_tree(np.random.default_rng(13), max_segments=9, max_len=200, forest=True)
    m, off, C = _maps(t)
    ch, w = 256, 4
    rng = np.random.default_rng(4)
    x = _dev(rng.standard_normal((C, ch)).astype(np.float32)).to(torch.bfloat16)
    dout = _dev(rng.standard_normal((C, ch)).astype(np.float32)).to(torch.bfloat16)
    wt = _dev(rng.standard_normal((ch, w)).astype(np.float32) / w)
    anc, goff, gl = harts.conv_tables(m, off, C, w)
    ancd, goffd, gld = _dev(anc), _dev(goff), _dev(gl)
    out, dx = torch.empty_like(x), torch.empty_like(x)
    dw = torch.empty((ch, w), device="cuda")
    ws = torch.empty(harts.conv_workspace_size(C, ch, w), dtype=torch.uint8, device="cuda")
    print(f"conv graph: C={C}", flush=True)

    def step():
        harts.conv_fwd(x, wt, ancd, out)
        harts.conv_bwd(x, wt, ancd, goffd, gld, dout, dx=dx, dweight=dw, workspace=ws)

    _replay_matches_eager(step, [out, dx, dw])


def test_logprob_graph_replay():
    C, V, S = 96, 4096, 500
    rng = np.random.default_rng(5)
    x = _dev(2.0 * rng.standard_normal((C, V)).astype(np.float32)).to(torch.bfloat16)
    m = rng.integers(0, C, size=S).astype(np.int64)
    lab = rng.integers(0, V, size=S).astype(np.int32)
    g = rng.standard_normal(S).astype(np.float32)
    md, ld, gd = _dev(m), _dev(lab), _dev(g)
    roff, rpos = harts.logprob_rows(m, C)
    roffd, rposd = _dev(roff), _dev(rpos)
    lp, lp2 = torch.empty(S, device="cuda"), torch.empty(S, device="cuda")
    q, q2 = torch.empty(C, dtype=torch.int32, device="cuda"), torch.empty(C, dtype=torch.int32, device="cuda")
    lse = torch.empty(C, device="cuda")
    dx = torch.empty_like(x)
    print(f"log-prob graph: C={C} V={V} S={S}", flush=True)

    def step():
        harts.logprob_gather(x, md, ld, lp, q=q, lse=lse)
        harts.logprob_backward(x, lse, roffd, rposd, ld, gd, dx)
        harts.logprob_gather_noalloc(x, md, ld, lp2, q=q2)

    _replay_matches_eager(step, [lp, q, lse, dx, lp2, q2])


def test_moe_graph_replay():
    C, E, k = 600, 128, 8
    rng = np.random.default_rng(6)
    z = _dev(2.0 * rng.standard_normal((C, E)).astype(np.float32))
    qn = rng.integers(1, 6, size=C).astype(np.int32)
    tq = _dev(qn)
    S = int(qn.sum())
    bias = _dev(0.01 * rng.standard_normal(E).astype(np.float32))
    top = torch.empty((C, k), dtype=torch.int32, device="cuda")
    lse = torch.empty(C, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    mass, losses = torch.empty(E, device="cuda"), torch.empty(2, device="cuda")
    dz = torch.empty_like(z)
    ws = torch.empty(harts.moe_workspace_size(C, E), dtype=torch.uint8, device="cuda")
    print(f"moe graph: C={C} E={E}", flush=True)

    def step():
        harts.moe_stats(z, tq, k, S, top, lse, counts, mass, losses, ws, bias=bias)
        harts.moe_grad(z, tq, counts, k, S, 0.7, 1.9, dz)

    _replay_matches_eager(step, [top, lse, counts, mass, losses, dz])
