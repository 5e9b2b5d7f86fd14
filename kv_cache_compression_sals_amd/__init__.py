"""SALS decode path and post-prefill KV compaction on MI355X (gfx950).

The computation lives in libsals.so (hand-written HIP kernels behind the C ABI declared in
include/sals.h); this package is its thin Python binding. Importing the binding needs torch;
loading the library happens on first use and fails loudly if it has not been built.
"""

from .binding import (  # noqa: F401
    SalsError,
    kv_compact,
    kv_compact_from_importance,
    kv_importance_budget,
    kv_importance_sparsity,
    kv_importance_sparsity_workspace_bytes,
    kv_layer_budgets,
    kv_outlier_importance,
    kv_outlier_importance_workspace_bytes,
    kv_quantize_mixed,
    kv_compact_workspace_bytes,
    n_selected,
    sals_decode_step,
    sals_decode_step_noalloc,
    sals_decode_step_threshold,
    sals_decode_step_traced,
    sals_decode_workspace_bytes,
    sals_dense_decode,
    sals_dense_decode_mixed,
    sals_dense_decode_mixed_workspace_bytes,
    sals_dense_decode_workspace_bytes,
    sals_project_kv,
    sals_reconstruct_kv,
)
