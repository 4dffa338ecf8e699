"""Plain reference for writing one new token's K and V into a paged KV cache.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may call this module; the product path never does.

What is computed: the decode step writes the new token's key and value rows
into the cache right before attention reads them ("rvLLM: High-performance LLM
inference in Rust", section "Kernel Compiler Stack", the per-layer decode
step list: the KV cache write follows RoPE and precedes attention), into a
paged cache held in f16 or FP8 (same page, sections "What's Inside" and
"Optional Features"; "Litellama", section "Features", FP8 KV cache).

For every sequence b with a position p = positions[b] inside its table
(0 <= p < 16 * max_blocks_per_seq) and a block id blk = block_table[b][p // 16]
inside the pool, and every KV head g and head-dim element d:

    k_cache[blk][g][d // X][p % 16][d % X] = enc(k_new[b][g][d], k_scale[g])
    v_cache[blk][g][d][p % 16]             = enc(v_new[b][g][d], v_scale[g])

(X = 16 / element bytes: the cache layout the decode kernels read). Any other
sequence writes nothing. enc is the identity on the storage bits when the
cache has the new rows' type; for an fp8 cache it is the quantizer of the
reading taken for the fp8 scales (per KV head, value = e4m3(code) * scale):

    code = RNE_e4m3(clamp(float32(x) / float32(scale), -448, 448))

with the division done in float32, ties to the even code, NaN to code 0x7F
and the sign kept (so -0 and tiny negatives give 0x80).
"""
import numpy as np

from .formats import E4M3_TABLE, ELEM_BYTES, decode
from .paged_decode import BLOCK_SIZE, page_x

# the non-negative finite E4M3 values, indexed by code 0 .. 126 (increasing)
_POS = E4M3_TABLE[:127]
assert np.all(np.diff(_POS) > 0)


def e4m3_encode(v):
    """float32 (or exactly representable float64) values -> E4M3 codes, by
    round-to-nearest, ties to the even code, after clamping to +-448; NaN ->
    0x7F; the sign bit follows the value's sign (including -0)."""
    v = np.atleast_1d(np.asarray(v, dtype=np.float64))
    nan = np.isnan(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), 448.0)
    hi = np.searchsorted(_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    exact = _POS[hi] == a
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    code[nan] = 0x7F
    return code


def widen_to_f32(raw, dtype):
    """Storage bits of f32 / f16 / bf16 values -> float32 (exact)."""
    return decode(raw, dtype).astype(np.float32)


def quantize_e4m3(raw, src_dtype, scale):
    """The fp8 cache codes of values stored as src_dtype, for one scale."""
    x = widen_to_f32(raw, src_dtype)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        y = (x / np.float32(scale)).astype(np.float32)
    return e4m3_encode(y)


def kv_append_ref(k_cache, v_cache, k_new, v_new, block_table, positions, src_dtype,
                  kv_dtype, k_scale=None, v_scale=None):
    """Return copies of (k_cache, v_cache) with the new rows written.

    k_new, v_new: storage arrays [B][Hkv][D] in src_dtype; caches in the layout
    above, kv_dtype == src_dtype or "fp8_e4m3" (with float32 k_scale, v_scale
    per KV head).
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    B, H, D = k_new.shape[:3]
    nb, mbs = k_out.shape[0], block_table.shape[1]
    X = page_x(kv_dtype)
    for b in range(B):
        p = int(positions[b])
        if p < 0 or p >= BLOCK_SIZE * mbs:
            continue
        blk = int(block_table[b, p // BLOCK_SIZE])
        if blk < 0 or blk >= nb:
            continue
        slot = p % BLOCK_SIZE
        for g in range(H):
            if kv_dtype == src_dtype:
                kr, vr = k_new[b, g], v_new[b, g]
            else:
                kr = quantize_e4m3(k_new[b, g], src_dtype, k_scale[g])
                vr = quantize_e4m3(v_new[b, g], src_dtype, v_scale[g])
            for d in range(D):
                k_out[blk, g, d // X, slot, d % X] = kr[d]
                v_out[blk, g, d, slot] = vr[d]
    return k_out, v_out


__all__ = ["e4m3_encode", "kv_append_ref", "quantize_e4m3", "widen_to_f32"]
assert ELEM_BYTES["fp8_e4m3"] == 1
