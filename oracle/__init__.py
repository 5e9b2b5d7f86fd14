"""CPU oracle for the SALS decode path and post-prefill KV compaction.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the C-ABI library and its Python binding) never imports, calls or links it,
and this package imports nothing from the product.

Plain, slow, fp64 NumPy. Each function follows one step of the method as the
pages state it (the SALS page, "方法详解 / 技术框架" stages 1-4 and "关键设计"
items 1-4; the VL-Cache author responses to reviewers KiPr W1/W2 and XVzL
W2/W3, and X8F2 Q2 for when eviction happens). Where the pages leave a step
open, the reading taken is written next to the code.

Pins (tests/test_oracle_pins.py) tie every function to something other than
itself: dense RoPE attention written with explicit loops, orthogonal/identity
projections, closed forms for uniform attention, a library softmax, brute-force
sorting, the complex-number form of RoPE and hand-worked selection examples.
No function here is "parity unpinned".
"""

from .sals import (  # noqa: F401
    attend_selected,
    decode_step,
    decode_step_threshold,
    group_of,
    kv_head_of,
    latent_query,
    latent_scores,
    project_kv,
    reconstruct,
    rope,
    rope_theta,
    select_tokens,
    select_tokens_threshold,
    stored_to_f64,
    topk_lowest_index,
)
from .compact import (  # noqa: F401
    compact_from_importance, dense_decode, energy_budgets, importance, importance_budget, kv_compact, layer_budgets,
    mass_budget, sparsity,
)
from .outlier import dct_basis, deviation_energy, lowpass, outlier_compact, outlier_importance  # noqa: F401
from .quant import dequantize_rows, mixed_decode, mixed_quantize, mixed_rows, quantize_group, quantize_rows  # noqa: F401
