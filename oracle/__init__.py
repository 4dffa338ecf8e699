"""Float64 CPU oracle for paged single-token decode attention.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the CPU
baseline leg of bench.py may import this package. It shares no code with the
HIP library (paged_kv_decode_05_amd) and imports nothing from it.

Parity pins: every function here is pinned by tests marked "not gpu" against
brute force on tiny inputs, a library attention routine, closed forms, and
invariants (see tests/test_oracle_pins.py); no function is parity-unpinned.
"""
from .formats import (E4M3_TABLE, ELEM_BYTES, STORAGE, decode, decode_bf16,
                      decode_e4m3, decode_f16, decode_f32, e4m3_value)
from .paged_decode import (BLOCK_SIZE, attend, gather_kv, lse_merge, page_x,
                           paged_decode_ref, paged_decode_split_ref)
from .kv_append import e4m3_encode, kv_append_ref, quantize_e4m3, widen_to_f32
from .shard_merge import shard_merge_ref
from .block_pool import BlockPoolRef, PoolError, chain_hash, fnv1a64
from .multi_query import multi_query_ref

__all__ = [
    "E4M3_TABLE", "ELEM_BYTES", "STORAGE", "decode", "decode_bf16",
    "decode_e4m3", "decode_f16", "decode_f32", "e4m3_value", "BLOCK_SIZE",
    "attend", "gather_kv", "lse_merge", "page_x", "paged_decode_ref",
    "paged_decode_split_ref", "e4m3_encode", "kv_append_ref", "quantize_e4m3",
    "widen_to_f32", "shard_merge_ref", "BlockPoolRef", "PoolError", "chain_hash", "fnv1a64",
    "multi_query_ref",
]
