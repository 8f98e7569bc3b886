"""Index-selected sparse attention on MI355X (gfx950).

The C ABI lives in libtis.so (see include/tis.h); this package holds its
ctypes binding (same entry-point names), the build step and the seeded
synthetic workload generators.
"""
from ._lib import (  # noqa: F401
    TIS_PHASE_DECODE, TIS_PHASE_PREFILL, TisError, Shape, make_shape, workspace_size,
    sparse_index_score, sparse_topk_select, paged_gather_attend, sparse_decode_step,
    paged_kv_append, abi_version, last_error,
)
