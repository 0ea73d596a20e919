"""RocketKV's hot path on MI355X (gfx950): SnapKV++ eviction and hybrid sparse decode attention.

The work runs in the HIP kernels of librkv.so behind the C ABI in include/rkv.h; this package is
its Python binding (torch tensors for device memory and streams).
"""
from .api import (  # noqa: F401
    RkvError,
    hybrid_decode_step,
    hybrid_decode_workspace_bytes,
    DECODE_STATUS_INVALID,
    decode_workspace_status,
    rkv_hybrid_decode_workspace,
    rkv_hybrid_decode_step,
    rkv_hybrid_decode_step_noalloc,
    rkv_build_page_summaries,
    rkv_build_page_summaries_cap,
    rkv_kv_append,
    rkv_hybrid_decode_step_cap,
    rkv_build_page_summaries_indexed,
    rkv_hybrid_decode_step_indexed,
    rkv_plan_budget,
    rkv_hybrid_approx_scores,
    rkv_snapkvpp_evict,
    rkv_sparse_attend_decode,
    rkv_topk_select,
    snapkvpp_workspace_bytes,
    sparse_attend_workspace_bytes,
    topk_workspace_bytes,
)
