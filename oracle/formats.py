"""Exact decoding of the storage formats the decode path reads, into float64.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module.

Formats:
  * "f32"  -- IEEE binary32, stored as float32.
  * "f16"  -- IEEE binary16, stored as 16-bit words.
  * "bf16" -- bfloat16 (the top half of a binary32), stored as 16-bit words.
  * "fp8_e4m3" -- the OCP 8-bit "E4M3" encoding, in the variant without
    infinities: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; the
    two codes S.1111.111 are NaN, every other code is finite, largest 448.
    The pages name this KV-cache format ("rvLLM: High-performance LLM inference
    in Rust", section "Optional Features", FP8 KV Cache; "Litellama", section
    "Features", FP8 KV Cache, and the "Quantization" table) without spelling
    out the variant; the OCP variant without infinities is the reading taken.

Every finite value of each format is exactly representable in float64, so the
decoders below are exact.
"""
import numpy as np

STORAGE = {
    "f32": np.float32,
    "f16": np.uint16,
    "bf16": np.uint16,
    "fp8_e4m3": np.uint8,
}

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}


def decode_f32(raw):
    return np.asarray(raw).view(np.float32).astype(np.float64)


def decode_f16(raw):
    return np.asarray(raw).view(np.uint16).view(np.float16).astype(np.float64)


def decode_bf16(raw):
    # bfloat16 is the high 16 bits of a binary32 word.
    words = np.asarray(raw).view(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # signalling-NaN words widen to NaN
        return words.view(np.float32).astype(np.float64)


def e4m3_value(code):
    """Value of one E4M3 code (0..255) from its bit fields."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:  # subnormal: no implicit leading one, exponent of 1 - bias
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(raw):
    return E4M3_TABLE[np.asarray(raw).view(np.uint8)]


DECODERS = {
    "f32": decode_f32,
    "f16": decode_f16,
    "bf16": decode_bf16,
    "fp8_e4m3": decode_e4m3,
}


def decode(raw, dtype):
    return DECODERS[dtype](raw)
