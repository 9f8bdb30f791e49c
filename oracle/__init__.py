"""FP64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library (no kernels,
headers, helpers, tables or pre/post-processing) and imports nothing from it.

Modules
-------
attend       plain float64 softmax attention gathered through the page table,
             the key-range partial form and the log-sum-exp merge
closed_forms the byte and block-count identities printed on the serving pages
paging       a plain model of the paged block allocator (sharing, copy-on-write,
             fenced release) and of appending new K/V rows to their pages
"""

from .attend import (  # noqa: F401
    bf16_bits_to_f64,
    gather_request_kv,
    attend_fp64,
    attend_key_range_fp64,
    combine_fp64,
)
from .closed_forms import (  # noqa: F401
    kv_bytes_per_token,
    blocks_needed,
    tail_waste,
    allocated_token_slots,
    kv_alloc_bytes,
    shared_prefix_alloc_bytes,
    shared_physical_blocks,
    block_references,
    causal_pairs,
    full_pairs,
    chunk_attention_flops,
)
