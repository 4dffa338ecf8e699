"""Pins for the shard-merge oracle (oracle/shard_merge.py): shards of every
sequence's positions, each attended on its own by the decode oracle, merge to
the unsharded decode; plus closed forms, shard-order invariance, empty shards
and NaN propagation. CPU only."""
import numpy as np
import pytest

import oracle
from paged_kv_decode_05_amd import workloads as W


def shard_bounds(L, S, align=16):
    """S contiguous, 16-aligned position ranges covering [0, L) (some may be empty)."""
    cuts = [min(L, -(-(L * s // S) // align) * align) for s in range(S)] + [L]
    return [(cuts[s], cuts[s + 1]) for s in range(S)]


def sharded_partials(wl, S):
    """Each shard's decode over its own positions (by the decode oracle, on a
    shifted block table): outputs [S, B, Hq, D] (float64) and lse [S, B, Hq]."""
    B = wl.q.shape[0]
    outs, lses = [], []
    for s in range(S):
        bt = np.zeros_like(wl.block_table)
        lens = np.zeros(B, dtype=np.int32)
        for b in range(B):
            lo, hi = shard_bounds(int(wl.context_lens[b]), S)[s]
            n = -(-hi // 16) - lo // 16
            bt[b, :n] = wl.block_table[b, lo // 16: lo // 16 + n]
            lens[b] = hi - lo
        o, l = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, bt, lens, wl.scale,
                                       wl.spec.io_dtype, wl.spec.kv_dtype, wl.k_scale, wl.v_scale,
                                       return_lse=True)
        outs.append(o)
        lses.append(l)
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("S", [1, 2, 3, 8])
def test_shards_merge_to_the_unsharded_decode(S):
    spec = W.small_variant(W.SPECS[5], 4, ("fixed", [20, 300, 1000, 2100]), max_blocks_per_seq=140)
    wl = W.make_workload(spec)
    outs, lses = sharded_partials(wl, S)
    B, Hq, D = outs.shape[1:]
    got, glse = oracle.shard_merge_ref(outs.reshape(S, B * Hq, D).astype(np.float32), lses.reshape(S, -1), "f32")
    want, wlse = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens,
                                         wl.scale, spec.io_dtype, spec.kv_dtype, return_lse=True)
    assert np.abs(got - want.reshape(B * Hq, D)).max() < 1e-6      # float32 shard outputs
    assert np.abs(glse - wlse.reshape(-1)).max() < 1e-12


def test_closed_forms_and_order_invariance():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((2, 3, 8)).astype(np.float32)
    # equal lse: the plain average; lse grows by ln 2
    out, lse = oracle.shard_merge_ref(o, np.full((2, 3), 0.7), "f32")
    assert np.allclose(out, (o[0].astype(np.float64) + o[1]) / 2, atol=1e-15)
    assert np.allclose(lse, 0.7 + np.log(2), atol=1e-15)
    # lse differing by ln 3: weights 3/4 and 1/4
    out, _ = oracle.shard_merge_ref(o, np.stack([np.full(3, np.log(3.0)), np.zeros(3)]), "f32")
    assert np.allclose(out, 0.75 * o[0].astype(np.float64) + 0.25 * o[1], atol=1e-15)
    # shard order does not matter
    o4 = rng.standard_normal((4, 5, 8)).astype(np.float32)
    l4 = rng.standard_normal((4, 5))
    a, la = oracle.shard_merge_ref(o4, l4, "f32")
    b, lb = oracle.shard_merge_ref(o4[::-1].copy(), l4[::-1].copy(), "f32")
    assert np.allclose(a, b, atol=1e-14) and np.allclose(la, lb, atol=1e-14)


def test_empty_shards_and_nan():
    o = np.ones((3, 2, 4), dtype=np.float32)
    o[1] *= 5
    lse = np.array([[0.2, -np.inf], [-np.inf, -np.inf], [-np.inf, np.nan]])
    out, l = oracle.shard_merge_ref(o, lse, "f32")
    assert np.array_equal(out[0], np.ones(4)) and l[0] == 0.2     # only shard 0 counts
    assert np.isnan(out[1]).all() and np.isnan(l[1])               # NaN in shard 2
    out, l = oracle.shard_merge_ref(o[:2], np.full((2, 2), -np.inf), "f32")
    assert np.array_equal(out, np.zeros((2, 4))) and np.all(np.isneginf(l))


def test_planted_mistake_is_caught():
    # merging with unnormalised weights (dropping the division) must fail the
    # unsharded comparison
    spec = W.small_variant(W.SPECS[3], 3, ("fixed", [40, 500, 900]), max_blocks_per_seq=60)
    wl = W.make_workload(spec)
    outs, lses = sharded_partials(wl, 3)
    w = np.exp(lses - lses.max(axis=0))
    wrong = (w[..., None] * outs).sum(axis=0)
    want = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens,
                                   wl.scale, spec.io_dtype, spec.kv_dtype)
    assert np.abs(wrong - want).max() > 1e-3
