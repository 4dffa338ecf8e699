"""Plain reference for merging decode-attention results of position shards.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may call this module; the product path never does.

What is computed: with decode context parallelism each shard attends over a
disjoint range of every sequence's positions, and the partial results are
combined by log-sum-exp ("RapidLLM", feature table, row "Decode context
parallelism"). For every row r (a (sequence, query head) pair) and shards
s = 0 .. S-1 with outputs o_s[r] and natural-log log-sum-exps lse_s[r]:

    M = max_s lse_s,  w_s = exp(lse_s - M),
    out[r] = sum_s w_s o_s[r] / sum_s w_s,   lse[r] = M + log sum_s w_s.

Readings taken where the page is silent: a shard with lse = -inf (no tokens)
contributes nothing, and a row with no contributing shard gives out = 0,
lse = -inf (as for an empty context); a NaN lse in any shard makes that row's
out and lse NaN (so an out-of-contract shard is never silently dropped).
"""
import numpy as np

from .formats import decode
from .paged_decode import lse_merge


def shard_merge_ref(shard_out, shard_lse, dtype):
    """shard_out: storage [S, rows, D] in dtype; shard_lse: [S, rows] (float32
    or float64, natural log). Returns (out [rows, D], lse [rows]) in float64."""
    outs = decode(np.asarray(shard_out), dtype)
    lses = np.asarray(shard_lse, dtype=np.float64)
    out, lse = lse_merge(outs, lses)
    bad = np.isnan(lses).any(axis=0)
    out = np.where(bad[:, None], np.nan, out)
    lse = np.where(bad, np.nan, lse)
    return out, lse


__all__ = ["shard_merge_ref"]
