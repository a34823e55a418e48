"""CLO decode-step hot path for AMD Instinct MI355X (gfx950).

The kernels and the C ABI live in libclo.so (include/clo.h); `clo` is its
Python binding (argument marshalling only), `hip_host` allocates pinned host
memory, `workload` lays out and loads one layer's buffers.
"""
from .clo import (  # noqa: F401
    CLO_BF16,
    CLO_F32,
    CloError,
    Layer,
    Shape,
    Sync,
    clo_decode_step,
    clo_gather_kv,
    clo_last_error,
    clo_reuse_select,
    clo_reuse_test,
    clo_sparse_attn,
    clo_status_string,
    clo_topk_select,
    clo_workspace_size,
    load,
)
