"""Float64 CPU oracle for grouped-query attention (GQA) over a KV cache.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY.  Only the test suite, the smoke
check and the bench's CPU-baseline leg may import this package.  The HIP
library never calls it, and it shares no code with the HIP path: the two meet
only in the seeded arrays that ``gqa_inputs`` produces.

What it computes is the plain definition of attention with the key/value
heads explicitly repeated along the query-head axis, in float64:

* ``attention``   decode and causal prefill outputs (and log-sum-exp);
* ``kv_math``     the closed forms for KV-cache bytes and decode FLOPs;
* ``paged``       decode over a paged KV cache (gather, then the plain definition);
* ``fp8``         decode over an E4M3 cache with per-KV-head scales (dequantise, then decode);
* ``backward``    gradients of causal prefill (repeat K/V, chain rule per head, sum back);
* ``wide``        decode whose cached rows are key and (leading columns) value: the absorbed-MLA shape.

Every function cites the passage of the source pages it follows.  The oracle
is pinned by tests/test_oracle_pins.py against values the pages print, closed
forms, exact special cases and a scalar brute force.
"""
from .attention import (  # noqa: F401
    group_size,
    kv_head_of,
    head_mapping,
    expand_kv_heads,
    softmax_average,
    decode,
    decode_one,
    prefill_causal,
    prefill_causal_rows,
)
from .paged import gather_pages, decode_paged  # noqa: F401
from .fp8 import e4m3_value, dequantize, decode_fp8  # noqa: F401
from .wide import decode_wide  # noqa: F401
from .backward import (  # noqa: F401
    reduce_kv_heads,
    prefill_causal_backward,
    prefill_causal_backward_group,
)
from .kv_math import (  # noqa: F401
    kv_cache_bytes,
    kv_bytes_per_token,
    decode_attention_flops,
    causal_prefill_flops,
    max_concurrent_requests,
)
