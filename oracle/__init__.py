"""fp64 CPU oracle for exact dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link
or execute anything in this package; only the tests, the smoke check and the
benchmark's CPU-baseline leg do. It shares no code with the HIP path.
"""
from .attention import (  # noqa: F401
    attention_head,
    attention_rows,
    attention_bhnd,
    attention_gqa,
    attention_varlen,
    online_attention_head,
    online_attention_head_fa1,
)
from .attention_bwd import attention_bwd_bhnd, attention_bwd_head, attention_bwd_sampled  # noqa: F401
from .schedule import varlen_lpt_order, varlen_tile_weights  # noqa: F401
