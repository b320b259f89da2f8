"""CPU float64 oracle for paged-attention decode (one or several new tokens per
sequence), prefill attention and the paged cache write.

TEST INFRASTRUCTURE ONLY: imported by `tests/`, `__graft_entry__.smoke()` and
the `cpu_baseline` leg of `bench.py`, never by the product path. It shares no
code with the HIP library or its binding.

Every function here is pinned by `-m "not gpu"` tests (brute force on tiny
inputs, closed forms, invariants, a library routine on expanded KV); none is
"parity unpinned".
"""
from .paged_attention import (  # noqa: F401
    BLOCK_SIZE,
    cache_write,
    gather_sequence,
    paged_decode,
    paged_decode_partitioned,
    paged_multi_query,
    prefill_attention,
    round_to_storage,
    widen,
)
