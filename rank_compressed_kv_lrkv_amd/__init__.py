"""LRKV compressed-cache attention for AMD Instinct MI355X (gfx950).

The compute lives in the C-ABI library ``lib/liblrkv.so`` (hand-written HIP
kernels); this package is its Python binding plus the seeded synthetic
workload generator used by the tests and the benchmark.
"""
from .binding import (  # noqa: F401
    DecodeCall, EXPORTED, LRKV_BF16, LRKV_F32, LrkvCache, LrkvError, decode_workspace, default_scale, library,
    lrkv_append, lrkv_cache_elems_per_token, lrkv_init, lrkv_decode, lrkv_decode_noalloc, lrkv_decode_scan_kernel, lrkv_decode_workspace_size,
    lrkv_decode_workspace_size_ex,
    lrkv_mha_decode, lrkv_mha_decode_workspace_size,
    lrkv_pack_projection, lrkv_prefill, lrkv_prefill_chunk, lrkv_prefill_kernel, lrkv_project_append, lrkv_project_kernel,
    lrkv_project_workspace_size, lrkv_status_string, lrkv_train_backward, lrkv_train_backward_workspace_size,
    lrkv_train_forward,
)
