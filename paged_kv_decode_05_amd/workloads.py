"""Seeded synthetic inputs for paged decode attention.

This module only draws and arranges inputs; it holds none of the attention
arithmetic. Both the HIP path (through the tests and bench.py) and the CPU
oracle are fed from it, so they see identical bits.

Recipe (per workload, all draws from one numpy Generator seeded with the
workload's seed, in this fixed order):
  1. context lengths: fixed list, integer-uniform with inclusive ends, or
     log-uniform L = floor(exp(U[ln lo, ln hi)));
  2. a permutation of the physical block pool;
  3. q, 4. the K pool, 5. the V pool: standard normal float32, then rounded to
     nearest-even into the storage type. For an fp8-e4m3 cache, each KV head
     gets scale = max|x| / 448 over that head's whole pool, and codes are
     round-to-nearest-even of clamp(x / scale, -448, 448).
Physical blocks are handed out from the permutation in (sequence, logical
block) order. With a shared prefix of S tokens, the first S/16 entries of the
permutation are the prefix blocks used by every sequence. Pool size is fixed
or ceil(ratio x blocks needed). The next unused block of the permutation is a
spare block filled with NaN; block-table entries past a sequence's last block
point at it, and every slot that no sequence reads as valid is NaN as well, so
a kernel that touches either shows NaN in its output.

Cache storage layout (what the shapes below mean; fixed by the library
header): k_cache [num_blocks][Hkv][D/x][16][x] with x = 16 / element bytes;
v_cache [num_blocks][Hkv][D][16].
"""
import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
FP8_MAX = 448.0
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F}


@dataclass(frozen=True)
class Spec:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    io_dtype: str                 # "f32" | "f16" | "bf16"
    kv_dtype: str                 # io_dtype or "fp8_e4m3"
    lens: Tuple                   # ("fixed", [..]) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    max_blocks_per_seq: int
    pool: Tuple                   # ("fixed", n) | ("ratio", r)
    partition_size: int           # 0 = single pass
    shared_prefix_tokens: int = 0
    seed: int = 0


# The five workloads. Seeds follow the workload number.
SPECS = {
    1: Spec("tiny_b4_h8kv2_d64_f32", 4, 8, 2, 64, "f32", "f32",
            ("fixed", [1, 17, 100, 256]), 16, ("fixed", 64), 0, 0, 1),
    2: Spec("qwen2.5-1.5b_b32_h12kv2_d128_f16", 32, 12, 2, 128, "f16", "f16",
            ("uniform", 256, 2048), 128, ("ratio", 1.2), 0, 0, 2),
    3: Spec("qwen2.5-7b_b32_h28kv4_d128_f16_split512", 32, 28, 4, 128, "f16", "f16",
            ("uniform", 512, 4096), 256, ("ratio", 1.2), 512, 0, 3),
    4: Spec("qwen2.5-7b_b128_h28kv4_d128_f16q_fp8kv_split512", 128, 28, 4, 128,
            "f16", "fp8_e4m3", ("uniform", 512, 4096), 256, ("ratio", 1.2), 512, 0, 4),
    5: Spec("llama3-8b_b8_h32kv8_d128_bf16_logu1k-128k_prefix4096_split512", 8, 32, 8,
            128, "bf16", "bf16", ("loguniform", 1024, 131072), 8192, ("ratio", 1.2),
            512, 4096, 5),
}


@dataclass
class Workload:
    spec: Spec
    context_lens: np.ndarray      # int32 [B]
    block_table: np.ndarray       # int32 [B, max_blocks_per_seq]
    num_blocks: int
    spare_block: int
    q: np.ndarray                 # storage [B, Hq, D]   (float32 or uint16 bits)
    k_cache: np.ndarray           # storage [nb, Hkv, D/x, 16, x]
    v_cache: np.ndarray           # storage [nb, Hkv, D, 16]
    scale: np.float32
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (fp8 only)
    v_scale: Optional[np.ndarray] = None

    @property
    def x(self):
        return 16 // ELEM_BYTES[self.spec.kv_dtype]

    def kv_bytes_logical(self):
        """K+V bytes of every (sequence, token, KV head) the call attends."""
        s = self.spec
        return int(self.context_lens.astype(np.int64).sum()) * 2 * s.num_kv_heads \
            * s.head_dim * ELEM_BYTES[s.kv_dtype]

    def kv_bytes_unique(self):
        """K+V bytes of distinct (physical block, slot, KV head) attended."""
        s = self.spec
        seen = {}
        for b in range(s.batch):
            L = int(self.context_lens[b])
            for j in range(-(-L // BLOCK_SIZE)):
                blk = int(self.block_table[b, j])
                seen[blk] = max(seen.get(blk, 0), min(BLOCK_SIZE, L - j * BLOCK_SIZE))
        return sum(seen.values()) * 2 * s.num_kv_heads * s.head_dim * ELEM_BYTES[s.kv_dtype]


def draw_lens(spec, rng):
    kind = spec.lens[0]
    if kind == "fixed":
        lens = np.array(spec.lens[1], dtype=np.int64)
        assert len(lens) == spec.batch
    elif kind == "uniform":
        lens = rng.integers(spec.lens[1], spec.lens[2], size=spec.batch, endpoint=True)
    elif kind == "loguniform":
        u = rng.uniform(math.log(spec.lens[1]), math.log(spec.lens[2]), size=spec.batch)
        lens = np.floor(np.exp(u)).astype(np.int64)
    else:
        raise ValueError(kind)
    assert lens.max() <= spec.max_blocks_per_seq * BLOCK_SIZE
    return lens.astype(np.int32)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _to_storage(x32, dtype):
    """Round float32 values to the storage type (nearest-even); return raw storage."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16) \
            .view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def _to_e4m3(x32, scale):
    import torch
    y = np.clip(x32 / np.float32(scale), -FP8_MAX, FP8_MAX).astype(np.float32)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _pool_draw(rng, shape, kv_dtype):
    """One KV pool: returns (storage, per-head scale or None)."""
    x32 = _normal(rng, shape)
    if kv_dtype != "fp8_e4m3":
        return _to_storage(x32, kv_dtype), None
    hkv = shape[1]
    scales = np.empty(hkv, dtype=np.float32)
    out = np.empty(shape, dtype=np.uint8)
    for g in range(hkv):
        scales[g] = np.float32(np.abs(x32[:, g]).max() / np.float32(FP8_MAX))
        out[:, g] = _to_e4m3(x32[:, g], scales[g])
    return out, scales


def _nan_fill(arr, dtype, index):
    if dtype == "f32":
        arr[index] = np.float32("nan")
    else:
        arr[index] = NAN_BITS[dtype]


def make_workload(spec, seed=None, poison=True):
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    B, Hq, Hkv, D = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    assert Hq % Hkv == 0 and D % 16 == 0
    x = 16 // ELEM_BYTES[spec.kv_dtype]

    lens = draw_lens(spec, rng)
    nblk = -(-lens.astype(np.int64) // BLOCK_SIZE)
    npre = spec.shared_prefix_tokens // BLOCK_SIZE
    needed = npre + int(np.maximum(nblk - npre, 0).sum())
    if spec.pool[0] == "fixed":
        pool = int(spec.pool[1])
    else:
        pool = int(math.ceil(spec.pool[1] * needed))
    assert pool >= needed + 1, "pool must leave room for the spare block"

    perm = rng.permutation(pool).astype(np.int32)
    table = np.empty((B, spec.max_blocks_per_seq), dtype=np.int32)
    nxt = npre
    for b in range(B):
        for j in range(int(nblk[b])):
            if j < npre:
                table[b, j] = perm[j]
            else:
                table[b, j] = perm[nxt]
                nxt += 1
    spare = int(perm[nxt])
    for b in range(B):
        table[b, int(nblk[b]):] = spare

    q = _to_storage(_normal(rng, (B, Hq, D)), spec.io_dtype)
    k_cache, k_scale = _pool_draw(rng, (pool, Hkv, D // x, BLOCK_SIZE, x), spec.kv_dtype)
    v_cache, v_scale = _pool_draw(rng, (pool, Hkv, D, BLOCK_SIZE), spec.kv_dtype)

    if poison:
        _nan_fill(k_cache, spec.kv_dtype, (spare,))
        _nan_fill(v_cache, spec.kv_dtype, (spare,))
        valid = {}
        for b in range(B):
            L = int(lens[b])
            for j in range(int(nblk[b])):
                blk = int(table[b, j])
                valid[blk] = max(valid.get(blk, 0), min(BLOCK_SIZE, L - j * BLOCK_SIZE))
        for blk, n in valid.items():
            if n < BLOCK_SIZE:
                _nan_fill(k_cache, spec.kv_dtype, (blk, slice(None), slice(None), slice(n, None)))
                _nan_fill(v_cache, spec.kv_dtype, (blk, slice(None), slice(None), slice(n, None)))

    return Workload(spec=spec, context_lens=lens, block_table=table, num_blocks=pool,
                    spare_block=spare, q=q, k_cache=k_cache, v_cache=v_cache,
                    scale=np.float32(1.0 / math.sqrt(D)), k_scale=k_scale, v_scale=v_scale)


def multi_query(wl, q_len, seed=None):
    """Query rows for q_len new tokens per sequence: storage [B][q_len][Hq][D]
    in the workload's io dtype, standard normal from a Generator seeded with
    (seed or the workload's seed) + 7919 * q_len. The workload's context
    lengths count the new tokens (their K/V are already in the cache)."""
    s = wl.spec
    rng = np.random.default_rng((s.seed if seed is None else seed) + 7919 * q_len)
    return _to_storage(_normal(rng, (s.batch, q_len, s.num_q_heads, s.head_dim)), s.io_dtype)


def small_variant(spec, batch, lens, max_blocks_per_seq=None, name_suffix="small"):
    """Same head shape and dtypes with a smaller batch and length mix."""
    mbs = max_blocks_per_seq
    if mbs is None:
        top = max(lens[1]) if lens[0] == "fixed" else lens[2]
        mbs = max(1, -(-top // BLOCK_SIZE))
    prefix = min(spec.shared_prefix_tokens, mbs * BLOCK_SIZE)
    return replace(spec, name=f"{spec.name}_{name_suffix}", batch=batch, lens=lens,
                   max_blocks_per_seq=mbs, shared_prefix_tokens=prefix)


# ---------------------------------------------------------------------------
# Upload to device tensors (storage bits unchanged).

def storage_tensor(raw, dtype):
    """A torch CPU tensor over the storage bits, typed for the binding."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == "f32":
        return t
    if dtype in ("f16", "bf16"):
        return t.view(torch.int16).view(torch.float16 if dtype == "f16" else torch.bfloat16)
    if dtype == "fp8_e4m3":
        return t.view(torch.uint8)
    raise ValueError(dtype)


def to_device(wl, device="cuda:0"):
    import torch
    s = wl.spec
    return {
        "q": storage_tensor(wl.q, s.io_dtype).to(device),
        "k_cache": storage_tensor(wl.k_cache, s.kv_dtype).to(device),
        "v_cache": storage_tensor(wl.v_cache, s.kv_dtype).to(device),
        "block_table": torch.from_numpy(wl.block_table).to(device),
        "context_lens": torch.from_numpy(wl.context_lens).to(device),
        "k_scale": None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(device),
        "v_scale": None if wl.v_scale is None else torch.from_numpy(wl.v_scale).to(device),
    }
