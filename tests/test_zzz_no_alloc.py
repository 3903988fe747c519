"""The no-allocation log-prob gather (harts_logprob_gather_noalloc, through the C ABI) against
harts_logprob_gather with a caller workspace on the same inputs: two calls in a row, the second
with fewer rows (the library's array still holds the first call's rows), each bit for bit and
within 1e-3 of the float64 definition; a row count above the maximum is refused."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import chunkwise_linear_attention_gated_amd as harts  # noqa: E402
from oracle import logprob as olp  # noqa: E402
from synthetic import tensors  # noqa: E402


def _case(C, V, seed, dtype):
    w = tensors.logprob_map(C, V, seed=seed)
    x = tensors.logits_torch(C, V, seed=seed, device="cuda", dtype=dtype)
    m = torch.from_numpy(w.m).cuda()
    lab = torch.from_numpy(w.labels).cuda()
    ref = torch.full((len(w.m),), float("nan"), device="cuda")
    q_ref = torch.full((C,), -1, dtype=torch.int32, device="cuda")
    harts.logprob_gather(x, m, lab, ref, q=q_ref,
                         workspace=torch.empty(harts.logprob_workspace_size(C), dtype=torch.uint8, device="cuda"))
    got = torch.full_like(ref, float("nan"))
    q = torch.full_like(q_ref, -1)
    harts.logprob_gather_noalloc(x, m, lab, got, q=q)
    torch.cuda.synchronize()
    assert torch.equal(got, ref) and torch.equal(q, q_ref)
    assert np.array_equal(q.cpu().numpy(), np.bincount(w.m, minlength=C).astype(np.int32))
    want = olp.logprob_rowwise(x.double().cpu(), w.m, w.labels)
    assert np.abs(got.cpu().numpy() - want).max() <= 1e-3


def test_noalloc_gather_equals_workspace_gather_twice():
    _case(4096, 32768, seed=11, dtype=torch.bfloat16)
    _case(777, 5003, seed=12, dtype=torch.float32)   # fewer rows, odd V (scalar tail)


def test_noalloc_gather_refuses_rows_above_the_maximum():
    C = (1 << 20) + 1
    x = torch.zeros((C, 1), device="cuda")
    m = torch.zeros(1, dtype=torch.int64, device="cuda")
    lab = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros(1, device="cuda")
    with pytest.raises(harts.HartsError) as e:
        harts.logprob_gather_noalloc(x, m, lab, out)
    assert "no-allocation maximum" in str(e.value)
