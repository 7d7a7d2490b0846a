"""fp64 CPU oracle for exact attention and its gradients (test infrastructure
only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library.
"""
from .exact import (  # noqa: F401
    admissible_mask,
    attention,
    attention_rows,
    attention_varlen,
    decode,
    head_attention,
    kv_head,
    weighted_values,
    merge_partials,
    scores,
    softmax_rows,
    tiled_online_attention,
    to_f64,
)
from .grad import (  # noqa: F401
    attention_grad,
    attention_grad_varlen,
    head_attention_grad,
    prob_grad,
    probabilities,
    softmax_backward,
)
from .kvcache import (  # noqa: F401
    bf16_bits,
    cache_row_index,
    gather_rows,
    kvcache_step,
    rotary,
    to_bf16_rne,
)
from .variants import (  # noqa: F401
    attention_ext,
    attention_ext_varlen,
    head_attention_ext,
    variant_scores,
    window_mask,
)
from .fp8 import (  # noqa: F401
    attention_fp8,
    attention_fp8_rounded_p,
    dequantize,
    e4m3_to_f64,
    p_rounding_bound,
    round_to_e4m3,
)
