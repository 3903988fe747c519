"""Tree-packed chunkwise gated-delta linear attention for MI355X (gfx950).

Thin Python binding over the C ABI declared in ``include/harts.h``
(``_harts.so``, built by :func:`build`).  Argument marshalling only: every
step of the path -- planning in C++, and every device operation in the HIP
kernels -- runs in the native library.  PyTorch supplies device memory and
the current HIP stream.  There is no fallback: if ``_harts.so`` is missing
the import of :mod:`chunkwise_linear_attention_gated_amd._lib` raises.
"""
from __future__ import annotations

from .build import build  # noqa: F401
from ._lib import (  # noqa: F401
    DTYPE_BF16, DTYPE_FP32, HartsError, TreePlan, VarlenPlan, DevicePlan, kda_fwd, kda_fwd_varlen, kda_bwd, logprob_gather,
    logprob_workspace_size, logprob_workspace, logprob_backward, logprob_rows, logprob_check_map, logprob_gather_noalloc, conv_tables, conv_workspace_size, conv_fwd,
    conv_bwd, attn_tables, attn_workspace_size, attn_fwd, attn_bwd, moe_workspace_size, moe_stats, moe_grad,
    moe_bias_update, library, version, profile_enable, profile_collect,
)
