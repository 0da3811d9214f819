"""MI355X (gfx950) absmax-scaled quantized linear layer.

* ``ql_*``: the C ABI of libqlinear.so (include/qlinear.h), one to one.
* ``quantize`` / ``qgemm`` / ``linear_forward`` / ...: the same calls on torch
  tensors (torch allocates the outputs and provides the stream).
* ``synth``: seeded synthetic inputs shaped like the pages' workloads.

Importing the package does not load the library; the first call does, and
fails loudly if it has not been built (``python -m
precision_quantized_gemm_amd.build``).
"""
from ._lib import (QL_DT_BF16, QL_DT_E4M3, QL_DT_FP32, QL_DT_INT32, QL_FMT_E4M3, QL_FMT_E5M2,
                   QL_FMT_INT8, QL_K_MAJOR, QL_MN_MAJOR, QL_PER_ROW, QL_PER_TENSOR, QLError,
                   ql_last_error, ql_linear_backward, ql_linear_forward, ql_linear_forward_noalloc, ql_linear_forward_static, ql_qgemm, ql_qgemm_batched, ql_quantize,
                   ql_quantize_groups, ql_quantize_ring, ql_status_string,
                   ql_workspace_bytes, ql_workspace_init)
from .api import (LinearGrads, LinearOut, linear_backward, linear_forward, linear_forward_static, new_workspace, qgemm,
                  qgemm_batched, quantize, quantize_groups, quantize_ring, workspace)

__all__ = [
    "ql_workspace_bytes", "ql_workspace_init", "ql_quantize", "ql_quantize_ring", "ql_qgemm", "ql_linear_forward",
    "ql_linear_forward_noalloc",
    "ql_linear_backward", "linear_backward", "LinearGrads", "ql_linear_forward_static", "linear_forward_static",
    "ql_quantize_groups", "ql_qgemm_batched", "quantize_groups", "qgemm_batched",
    "ql_status_string", "ql_last_error", "QLError",
    "quantize", "quantize_ring", "qgemm", "linear_forward", "LinearOut", "workspace", "new_workspace",
    "QL_FMT_E4M3", "QL_FMT_E5M2", "QL_FMT_INT8", "QL_DT_BF16", "QL_DT_FP32", "QL_DT_E4M3",
    "QL_DT_INT32", "QL_PER_TENSOR", "QL_PER_ROW", "QL_K_MAJOR", "QL_MN_MAJOR",
]
