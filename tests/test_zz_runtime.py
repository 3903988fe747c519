"""The library shares PyTorch's HIP runtime: importing the binding in a fresh
process, before torch, must still let device calls see the GPU."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_binding_first_import_order():
    code = ("import numpy as np, chunkwise_linear_attention_gated_amd as h, torch;"
            "p = h.TreePlan(np.array([1,2,3],np.int32), np.array([0,3],np.int64), 16);"
            "d = h.DevicePlan(p, 2, 16, 16, h.DTYPE_FP32); print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]
