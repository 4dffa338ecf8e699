"""Plain float64 reference for attention of several new query tokens per
sequence over a paged KV cache, causal among the new tokens.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may call this module; the product path never does.

What is computed: the attention step of chunked prefill and of speculative
verification, where each sequence brings T new tokens at once instead of one
("Litellama", section "Features": Chunked Prefill splits long prompts into
512-token chunks that interleave with decode requests, and section
"Architecture": flash-attention kernels over unpadded sequences with GQA;
"rvLLM: High-performance LLM inference in Rust", section on speculative
decoding: the target model verifies several drafted tokens per step). The
new tokens' K and V are already in the cache (appended first, as for a
single token), so the sequence's cached length L counts them: new token t
(t = 0 .. T-1) sits at position L - T + t and, causally, sees positions
0 .. L - T + t. For every sequence b, new token t and query head h (KV head
g = h // (Hq / Hkv)):

    n     = L - T + t + 1        (visible tokens; none when n <= 0)
    s_j   = scale * <q[b,t,h,:], k_j>                  j = 0 .. n-1
    out   = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s)
    lse   = max s + log sum_j exp(s_j - max s)         (natural log)

with k_j, v_j found through the block table as for single-token decode.

Readings taken where the pages are silent (each listed in the design notes):
  * q and out are [B][T][Hq][D], lse is [B][T][Hq]; one T for the whole call;
  * a token with no visible position (L < T, the leading padding of a short
    sequence) gets out = 0 and lse = -inf, as an empty sequence does;
  * with T = 1 this is single-token decode exactly.
"""
import numpy as np

from .formats import decode
from .paged_decode import BLOCK_SIZE, attend, gather_kv


def multi_query_ref(q, k_cache, v_cache, block_table, context_lens, scale, io_dtype,
                    kv_dtype, k_scale=None, v_scale=None, return_lse=False, seqs=None):
    """Float64 attention of T new tokens per sequence over the paged cache.

    q            raw storage [B, T, Hq, D] in io_dtype
    k_cache, v_cache, block_table, context_lens, scale, k_scale, v_scale:
                 as for paged_decode_ref (context_lens count the new tokens)
    seqs         optional subset of sequence indices to compute

    Returns out float64 [B, T, Hq, D] (sequences not in `seqs` are NaN), and
    lse float64 [B, T, Hq] when return_lse.
    """
    qv = decode(q, io_dtype)
    B, T, Hq, D = qv.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.full((B, T, Hq, D), np.nan)
    lse = np.full((B, T, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        nblk = -(-L // BLOCK_SIZE)
        blocks = np.asarray(block_table[b, :nblk], dtype=np.int64)
        for g in range(Hkv):
            k_rows, v_rows = gather_kv(k_cache, v_cache, blocks, g, L, kv_dtype)
            if kv_dtype == "fp8_e4m3":
                k_rows = k_rows * float(np.float32(k_scale[g]))
                v_rows = v_rows * float(np.float32(v_scale[g]))
            for t in range(T):
                n = max(L - T + t + 1, 0)
                o, l = attend(qv[b, t, g * G:(g + 1) * G], k_rows[:n], v_rows[:n], scale64)
                out[b, t, g * G:(g + 1) * G] = o
                lse[b, t, g * G:(g + 1) * G] = l
    return (out, lse) if return_lse else out


__all__ = ["multi_query_ref"]
