"""Plain float64 reference for single-token decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may call this module; the product path never does.

What is computed (the pages never write the formula; this is the plain
reading of the decode attention they describe):
  * "rvLLM: High-performance LLM inference in Rust", section "Kernel Compiler
    Stack": the decode-attention kernel does an online softmax over a paged KV
    cache with grouped-query heads, and runs right after the step that writes
    the new token's K/V into the cache.
  * "Welcome to vLLM" (feature list) and "Litellama" ("Features": attention
    backends for unpadded sequences with GQA; "Architecture": per-step KV
    bookkeeping handed to the kernels, PagedAttention over the KV pool).
For every sequence b and query head h, with g the KV head of h and L the
sequence's cached length:

    s_t   = scale * <q[b,h,:], k_t>                     t = 0 .. L-1
    out   = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)
    lse   = max s + log sum_t exp(s_t - max s)          (natural log)

where k_t, v_t are token t's key and value rows for head g, found through the
block table: block = block_table[b, t // 16], slot = t % 16.  Online softmax,
split-K partitions and the log-sum-exp merge are exact rewrites of this same
result, so the reference computes only the definition above.
`paged_decode_split_ref` restates the log-sum-exp merge ("RapidLLM", feature
table, row "Decode context parallelism": partial attention over disjoint KV
ranges merged by log-sum-exp) so that tests can check the identity the
kernels rely on.

Readings taken where the pages are silent (each listed in the design notes):
  * query head h uses KV head g = h // (Hq / Hkv) (contiguous groups);
  * scale is the float32 value the kernel receives, widened exactly;
  * K and V pages are [16 tokens x D] per (block, KV head), stored as
        k_cache[num_blocks][Hkv][D // x][16][x],  x = 16 / element bytes
        v_cache[num_blocks][Hkv][D][16]
    (the layout chosen for the kernels; the pages give none);
  * slots at or past L, and block-table entries past the last used block,
    are never read;
  * L = 0 gives out = 0 and lse = -inf;
  * fp8 KV: value = e4m3(code) * k_scale[g] (resp. v_scale[g]).
"""
import numpy as np

from .formats import ELEM_BYTES, decode

BLOCK_SIZE = 16


def page_x(kv_dtype):
    """Elements per 16-byte group in the K page layout."""
    return 16 // ELEM_BYTES[kv_dtype]


def gather_kv(k_cache, v_cache, blocks, g, L, kv_dtype):
    """Rows of K and V (float64, [L, D]) for KV head g over the given blocks.

    blocks: physical block ids of logical blocks 0 .. ceil(L/16)-1.
    """
    nblk = len(blocks)
    x = page_x(kv_dtype)
    kp = decode(k_cache[blocks, g], kv_dtype)          # [nblk, D/x, 16, x]
    D = kp.shape[1] * kp.shape[3]
    k_rows = kp.transpose(0, 2, 1, 3).reshape(nblk * BLOCK_SIZE, D)
    vp = decode(v_cache[blocks, g], kv_dtype)          # [nblk, D, 16]
    v_rows = vp.transpose(0, 2, 1).reshape(nblk * BLOCK_SIZE, D)
    assert x * kp.shape[1] == D
    return k_rows[:L], v_rows[:L]


def attend(q64, k_rows, v_rows, scale64):
    """Softmax attention of query rows q64 [G, D] over k_rows/v_rows [L, D].

    Returns (out [G, D], lse [G]) in float64; L = 0 gives zeros and -inf.
    """
    G, D = q64.shape
    L = k_rows.shape[0]
    if L == 0:
        return np.zeros((G, D)), np.full(G, -np.inf)
    s = scale64 * (q64 @ k_rows.T)                      # [G, L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    denom = e.sum(axis=1)
    out = (e @ v_rows) / denom[:, None]
    lse = m[:, 0] + np.log(denom)
    return out, lse


def _heads(q, io_dtype):
    return decode(q, io_dtype)                          # [B, Hq, D]


def paged_decode_ref(q, k_cache, v_cache, block_table, context_lens, scale,
                     io_dtype, kv_dtype, k_scale=None, v_scale=None,
                     return_lse=False, seqs=None):
    """Float64 decode attention over the paged cache.

    q            raw storage [B, Hq, D] in io_dtype ("f32" | "f16" | "bf16")
    k_cache      raw storage [num_blocks, Hkv, D/x, 16, x] in kv_dtype
    v_cache      raw storage [num_blocks, Hkv, D, 16] in kv_dtype
    block_table  int [B, max_blocks_per_seq]
    context_lens int [B]
    scale        softmax scale; taken as float32, then widened exactly
    k_scale/v_scale  float32 [Hkv], used only for kv_dtype "fp8_e4m3"
    seqs         optional subset of sequence indices to compute

    Returns out float64 [B, Hq, D] (rows of sequences not in `seqs` are NaN),
    and lse float64 [B, Hq] when return_lse.
    """
    qv = _heads(q, io_dtype)
    B, Hq, D = qv.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        nblk = -(-L // BLOCK_SIZE)
        blocks = np.asarray(block_table[b, :nblk], dtype=np.int64)
        for g in range(Hkv):
            k_rows, v_rows = gather_kv(k_cache, v_cache, blocks, g, L, kv_dtype)
            if kv_dtype == "fp8_e4m3":
                k_rows = k_rows * float(np.float32(k_scale[g]))
                v_rows = v_rows * float(np.float32(v_scale[g]))
            o, l = attend(qv[b, g * G:(g + 1) * G], k_rows, v_rows, scale64)
            out[b, g * G:(g + 1) * G] = o
            lse[b, g * G:(g + 1) * G] = l
    return (out, lse) if return_lse else out


def lse_merge(outs, lses):
    """Merge partial results of disjoint KV ranges by log-sum-exp.

    outs [P, ..., D], lses [P, ...]: each partial is softmax attention over its
    own range (a range with no tokens has lse = -inf and contributes nothing).
    With M = max_p lse_p and w_p = exp(lse_p - M):
        out = sum_p w_p out_p / sum_p w_p,   lse = M + log sum_p w_p.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Ms), 0.0)
    wsum = w.sum(axis=0)
    safe = np.where(wsum > 0, wsum, 1.0)
    out = (w[..., None] * outs).sum(axis=0) / safe[..., None]
    out = np.where((wsum > 0)[..., None], out, 0.0)
    lse = np.where(wsum > 0, Ms + np.log(safe), -np.inf)
    return out, lse


def paged_decode_split_ref(q, k_cache, v_cache, block_table, context_lens,
                           scale, io_dtype, kv_dtype, partition_size,
                           k_scale=None, v_scale=None):
    """Same result computed as split-K partitions merged by log-sum-exp.

    Partition p of a sequence covers tokens [p*partition_size,
    min((p+1)*partition_size, L)).  Each partition is attended on its own,
    then the partials are merged with `lse_merge`.  Returns (out, lse).
    """
    qv = _heads(q, io_dtype)
    B, Hq, D = qv.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        L = int(context_lens[b])
        nblk = -(-L // BLOCK_SIZE)
        blocks = np.asarray(block_table[b, :nblk], dtype=np.int64)
        P = max(1, -(-L // partition_size))
        for g in range(Hkv):
            k_rows, v_rows = gather_kv(k_cache, v_cache, blocks, g, L, kv_dtype)
            if kv_dtype == "fp8_e4m3":
                k_rows = k_rows * float(np.float32(k_scale[g]))
                v_rows = v_rows * float(np.float32(v_scale[g]))
            parts_o, parts_l = [], []
            for p in range(P):
                lo, hi = p * partition_size, min((p + 1) * partition_size, L)
                o, l = attend(qv[b, g * G:(g + 1) * G], k_rows[lo:hi],
                              v_rows[lo:hi], scale64)
                parts_o.append(o)
                parts_l.append(l)
            o, l = lse_merge(parts_o, parts_l)
            out[b, g * G:(g + 1) * G] = o
            lse[b, g * G:(g + 1) * G] = l
    return out, lse
