"""Seeded input generators: reproducibility, pool rule, block assignment,
shared prefix and NaN poisoning."""
import math

import numpy as np
import pytest

from paged_kv_decode_05_amd import workloads as W


def small(k, batch=6):
    s = W.SPECS[k]
    lens = {1: s.lens, 2: ("uniform", 16, 300), 3: ("uniform", 100, 700),
            4: ("uniform", 100, 700), 5: ("loguniform", 20, 2000)}[k]
    if k == 1:
        return s
    return W.small_variant(s, batch, lens)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_reproducible_and_seed_sensitive(k):
    a, b = W.make_workload(small(k)), W.make_workload(small(k))
    for f in ("context_lens", "block_table", "q", "k_cache", "v_cache"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=False) or \
            np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8))
    c = W.make_workload(small(k), seed=1234)
    assert not np.array_equal(a.q.view(np.uint8), c.q.view(np.uint8))


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_pool_and_block_assignment(k):
    wl = W.make_workload(small(k))
    s = wl.spec
    nblk = -(-wl.context_lens.astype(int) // 16)
    npre = s.shared_prefix_tokens // 16
    needed = npre + int(np.maximum(nblk - npre, 0).sum())
    assert wl.num_blocks == math.ceil(1.2 * needed)
    used = set()
    for b in range(s.batch):
        row = wl.block_table[b]
        for j in range(nblk[b]):
            if j >= npre:
                assert row[j] not in used     # private blocks are never shared
                used.add(int(row[j]))
        assert (row[nblk[b]:] == wl.spare_block).all()
        assert (row[:nblk[b]] < wl.num_blocks).all() and (row[:nblk[b]] >= 0).all()
    assert wl.spare_block not in used


def test_tiny_workload_exact_sizes():
    wl = W.make_workload(W.SPECS[1])
    assert list(wl.context_lens) == [1, 17, 100, 256]
    assert wl.num_blocks == 64 and wl.block_table.shape == (4, 16)
    assert wl.kv_bytes_logical() == 382976
    assert wl.scale == np.float32(1 / 8)


def test_shared_prefix_blocks():
    spec = W.small_variant(W.SPECS[5], 5, ("fixed", [50, 4096, 5000, 4100, 16]),
                           max_blocks_per_seq=320)
    wl = W.make_workload(spec)
    assert spec.shared_prefix_tokens == 4096
    pre = wl.block_table[1, :256]
    assert len(set(pre.tolist())) == 256
    assert np.array_equal(wl.block_table[2, :256], pre)
    assert np.array_equal(wl.block_table[0, :4], pre[:4])
    assert wl.block_table[4, 0] == pre[0]
    assert wl.kv_bytes_unique() < wl.kv_bytes_logical()


def test_fp8_scales_are_per_head_amax():
    wl = W.make_workload(small(4))
    assert wl.k_scale.shape == (4,) and wl.v_scale.shape == (4,)
    import oracle
    k = oracle.decode(wl.k_cache, "fp8_e4m3")
    for g in range(4):
        kk = k[:, g]
        kk = kk[np.isfinite(kk)]
        assert np.abs(kk).max() == 448.0     # the amax element lands on the top code
    assert wl.k_scale.dtype == np.float32


def test_poison_marks_unread_slots_only():
    spec = W.small_variant(W.SPECS[3], 4, ("fixed", [17, 32, 5, 600]))
    wl = W.make_workload(spec)
    import oracle
    k = oracle.decode(wl.k_cache, "f16")
    v = oracle.decode(wl.v_cache, "f16")
    blk = wl.block_table[0, 1]          # second block of a 17-token sequence: slot 0 valid
    assert np.isfinite(k[blk, :, :, 0]).all() and np.isnan(k[blk, :, :, 1:]).all()
    assert np.isfinite(v[blk, :, :, 0]).all() and np.isnan(v[blk, :, :, 1:]).all()
    blk = wl.block_table[1, 1]          # 32 tokens: full block
    assert np.isfinite(k[blk]).all()
    assert np.isnan(k[wl.spare_block]).all()
