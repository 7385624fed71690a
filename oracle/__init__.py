"""Plain CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
check and the CPU-baseline leg of the benchmark may import anything in
this package.  The GPU library never calls it, and it never calls the GPU
library: the two share no code.  Every value here is computed in float64
(numpy) from host arrays whose bits equal the device tensors.

Sources cited in the modules below (titles of the three pages this work
follows; section names are quoted as headings on those pages):

* [TEQ]  "Your GPU was mostly empty: how PagedAttention turned KV-cache
         waste into 2-4x throughput" (blog.teqners.com).
* [IV]   "vLLM and PagedAttention" (interviewsvector.com), a summary of
         "Efficient Memory Management for Large Language Model Serving
         with PagedAttention" (Kwon et al.).
* [AITJ] "PagedAttention KV cache memory management" (aitechjournal.org).
* [VAS]  Vaswani et al., "Attention Is All You Need", 2017, eq. (1):
         scaled dot-product attention.  The pages name attention but never
         write its formula; this is the textbook definition they rely on.

Parity status of every function is stated in its module header.  All
functions here are pinned by tests against the pages' worked numbers,
closed forms, invariants or brute force; none is "parity unpinned".
"""

from .formats import to_f64, bits_view  # noqa: F401
from .paged_attention import (  # noqa: F401
    gather_sequence_kv,
    decode_attention,
    decode_attention_partitioned,
    attention_one_head,
)
from .cache_ops import reshape_and_cache, copy_blocks, reshape_and_cache_fp8  # noqa: F401
from .prefill import prefill_attention  # noqa: F401
from .fp8 import e4m3_decode, e4m3_encode, quantize as e4m3_quantize  # noqa: F401
from .kv_accounting import (  # noqa: F401
    kv_bytes_per_token,
    kv_bytes_per_token_layer,
    sequence_cache_bytes,
    blocks_needed,
    empty_slots,
    waste_fraction,
)
