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
