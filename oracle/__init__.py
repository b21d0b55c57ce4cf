"""fp64 CPU oracle for the paged KV-cache data plane.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library.  It shares no code
with the HIP path.  ``fp64`` holds the NumPy definition, ``brute`` a
pure-Python scalar version for tiny shapes.
"""
from .fp64 import (  # noqa: F401
    attention, bf16_to_f64, block_fill, blocks_for, check_store_targets, kv_head_of,
    logical_block, paged_decode, paged_prefill, slot_of, softmax_weights, store_kvcache,
    visible_keys,
)
