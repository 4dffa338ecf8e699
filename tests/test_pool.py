"""The native block pool (pa_pool_* in libpadecode.so) against the oracle's
BlockPoolRef: the same operations in the same order must give the same block
ids, the same cached-token counts, the same failures (with nothing changed),
the same free-queue size and the same block tables. Host code only: CPU."""
import os
import random

import numpy as np
import pytest

import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import _lib
from oracle import BlockPoolRef, PoolError

pytestmark = pytest.mark.skipif(not os.path.exists(pkd.library_path()),
                                reason="libpadecode.so not built")


class Pair:
    """Drives the native pool and the oracle side by side and compares them
    after every operation."""

    def __init__(self, num_blocks, seed):
        self.nat = pkd.BlockPool(num_blocks, seed)
        self.ref = BlockPoolRef(num_blocks, seed)
        self.mbs = num_blocks

    def _both(self, nat_fn, ref_fn):
        try:
            want, want_err = ref_fn(), None
        except PoolError as e:
            want, want_err = None, e
        try:
            got, got_err = nat_fn(), None
        except pkd.PaError as e:
            got, got_err = None, e
        assert (want_err is None) == (got_err is None), (want_err, got_err)
        if got_err is not None:
            assert got_err.status in (_lib.PA_ERR_CAPACITY, _lib.PA_ERR_STATE, 2)
        assert got == want
        self.compare()
        return want_err is None

    def add(self, sid, tokens):
        return self._both(lambda: self.nat.add_sequence(sid, tokens),
                          lambda: self.ref.add_sequence(sid, tokens))

    def append(self, sid, tok):
        return self._both(lambda: self.nat.append_token(sid, tok),
                          lambda: self.ref.append_token(sid, tok))

    def free(self, sid):
        return self._both(lambda: self.nat.free_sequence(sid),
                          lambda: self.ref.free_sequence(sid))

    def compare(self):
        assert self.nat.num_free() == self.ref.num_free()
        sids = sorted(self.ref.seqs)
        if not sids:
            return
        rows, lens = self.ref.block_table(sids, self.mbs, -1)
        table, got_lens = self.nat.block_table(sids, self.mbs, -1)
        assert table.tolist() == rows
        assert got_lens.tolist() == lens
        # the shared prefix of the whole set and of a few subsets
        rnd = random.Random(len(sids) * 31 + int(self.nat.num_free()))
        subsets = [sids] + [rnd.sample(sids, rnd.randint(1, len(sids))) for _ in range(3)]
        for sub in subsets:
            assert self.nat.shared_prefix(sub) == expected_shared_prefix(self.ref, sub), sub


def expected_shared_prefix(ref, sids):
    """The definition, tried for every P from the largest down: each
    sequence holds the longest one's blocks at each of its own full blocks
    below P (the longest: the first among equals in `sids`)."""
    if not sids:
        return 0
    longest = sids[0]
    for sid in sids:
        if len(ref.seqs[sid]["tokens"]) > len(ref.seqs[longest]["tokens"]):
            longest = sid
    top = ref.seqs[longest]
    for P in range(len(top["tokens"]) // 16, -1, -1):
        if all(ref.seqs[sid]["blocks"][j] == top["blocks"][j]
               for sid in sids for j in range(min(P, len(ref.seqs[sid]["tokens"]) // 16))):
            return P
    return 0


def test_hand_worked_scenario_matches():
    p = Pair(6, 7)
    assert p.add(1, list(range(40)))
    assert p.add(2, list(range(32)) + list(range(100, 110)))
    assert p.nat.block_table([2], 4)[0].tolist() == [[0, 1, 3, 0]]
    assert p.free(1)
    assert p.add(3, list(range(500, 532)))
    for tok in range(110, 117):
        assert p.append(2, tok)
    assert not p.add(4, list(range(16)) + [1, 2, 3])          # out of blocks
    assert p.free(3)
    assert p.add(4, list(range(16)) + [1, 2, 3])
    assert p.nat.block_table([4], 2)[0].tolist() == [[0, 5]]
    assert not p.add(5, list(range(500, 532)))                # needs 2, has 1


def test_cached_token_counts():
    p = pkd.BlockPool(64, 3)
    pre = list(range(1000, 1064))                             # four blocks
    assert p.add_sequence(0, pre + [1, 2, 3]) == 0
    assert p.add_sequence(1, pre + [9]) == 64
    assert p.add_sequence(2, pre[:40]) == 32                  # two full blocks, then partial
    assert p.add_sequence(3, []) == 0
    assert p.block_table([3], 1, -7)[0].tolist() == [[-7]]


def test_error_statuses_and_nothing_written():
    p = pkd.BlockPool(4, 0)
    p.add_sequence(5, list(range(20)))
    with pytest.raises(pkd.PaError) as e:
        p.add_sequence(5, [1])
    assert e.value.status == _lib.PA_ERR_STATE
    for fn in (lambda: p.append_token(6, 1), lambda: p.free_sequence(6)):
        with pytest.raises(pkd.PaError) as e:
            fn()
        assert e.value.status == _lib.PA_ERR_STATE
    with pytest.raises(pkd.PaError) as e:
        p.add_sequence(7, list(range(100, 148)))
    assert e.value.status == _lib.PA_ERR_CAPACITY and p.num_free() == 2
    lib = _lib.load_library()
    table = np.full((2, 1), 99, dtype=np.int32)
    ids = np.array([5, 5], dtype=np.int64)
    assert lib.pa_pool_block_table(p._h, ids.ctypes.data, 2, 1, 0, table.ctypes.data,
                                   None) == 2          # two blocks do not fit one column
    assert table.tolist() == [[99], [99]]
    ids = np.array([5, 8], dtype=np.int64)
    assert lib.pa_pool_block_table(p._h, ids.ctypes.data, 2, 4, 0, table.ctypes.data,
                                   None) == _lib.PA_ERR_STATE
    for tok in range(12):
        p.append_token(5, tok)                                 # 32 tokens: two blocks
    p.append_token(5, 1)                                       # third block
    p.append_token(5, 2)
    p.add_sequence(9, list(range(200, 216)))                   # the last free block
    with pytest.raises(pkd.PaError) as e:
        for tok in range(30):
            p.append_token(5, tok)
    assert e.value.status == _lib.PA_ERR_CAPACITY
    assert p.block_table([5], 4)[1].tolist() == [48]           # 34 + 14 accepted


def test_shared_prefix_of_requests_behind_common_prompts():
    pool = pkd.BlockPool(200, 3)
    base = list(range(100, 164))                     # 64 tokens: 4 full blocks
    pool.add_sequence(0, base + [1, 2, 3])           # 4 full blocks + 3 tokens
    pool.add_sequence(1, base + [7] * 20)            # shares 4 blocks, 5 full
    pool.add_sequence(2, base[:40])                  # shares 2 full blocks, private partial third
    pool.add_sequence(3, list(range(500, 540)))      # nothing shared
    pool.add_sequence(4, base[:48] + [9] * 30)       # shares 3 blocks, its 4th full block differs
    # the longest (1) has 5 full blocks; 0 uses 4 of them, all shared
    assert pool.shared_prefix([0, 1]) == 5
    assert pool.shared_prefix([0, 1, 2]) == 5        # 2 agrees on its 2 full blocks
    assert pool.shared_prefix([2]) == 2
    assert pool.shared_prefix([0, 1, 4]) == 3        # 4 differs at its block 3
    assert pool.shared_prefix([0, 1, 3]) == 0
    assert pool.shared_prefix([]) == 0
    with pytest.raises(pkd.PaError) as e:
        pool.shared_prefix([0, 99])
    assert e.value.status == _lib.PA_ERR_STATE
    pool.close()


def test_null_and_shape_arguments():
    lib = _lib.load_library()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.pa_pool_create(0, 1, ctypes.byref(h)) == 2 and not h.value
    assert lib.pa_pool_create(4, 1, None) == 1
    assert lib.pa_pool_add_sequence(None, 1, None, 0, None) == 1
    assert lib.pa_pool_append_token(None, 1, 1) == 1
    assert lib.pa_pool_free_sequence(None, 1) == 1
    assert lib.pa_pool_num_free(None) == -1
    assert lib.pa_pool_block_table(None, None, 0, 1, 0, None, None) == 1
    lib.pa_pool_destroy(None)
    p = pkd.BlockPool(4, 1)
    assert lib.pa_pool_add_sequence(p._h, 1, None, 3, None) == 1
    assert lib.pa_pool_add_sequence(p._h, 1, None, -1, None) == 2
    assert lib.pa_pool_block_table(p._h, None, 0, 0, 0, None, None) == 2
    assert lib.pa_pool_block_table(p._h, None, 0, 1, 0, None, None) == 0


@pytest.mark.parametrize("seed", range(6))
def test_random_operation_sequences_match_the_oracle(seed):
    """Prompts drawn from a few shared prefixes (prefix hits, shared blocks),
    appended tokens from a 3-token vocabulary (sequences complete identical
    blocks, so a key is often cached already), a pool small enough that adds
    and appends fail and cached blocks get evicted, and operations on unknown
    or existing ids."""
    rnd = random.Random(seed)
    nb = rnd.choice([12, 24, 40])
    p = Pair(nb, seed * 7919)
    prefixes = [[rnd.randrange(50) for _ in range(rnd.choice([16, 32, 48, 20]))]
                for _ in range(3)]
    next_id = 0
    live = []
    for _ in range(600):
        r = rnd.random()
        if r < 0.3 or not live:
            toks = list(rnd.choice(prefixes)) if rnd.random() < 0.7 else []
            toks = toks[: rnd.randrange(len(toks) + 1)] if rnd.random() < 0.3 else toks
            toks += [rnd.randrange(3) for _ in range(rnd.randrange(0, 40))]
            sid = next_id if rnd.random() < 0.95 or not live else rnd.choice(live)
            if p.add(sid, toks):
                live.append(sid)
            next_id += sid == next_id
        elif r < 0.8:
            sid = rnd.choice(live) if rnd.random() < 0.97 else -5
            p.append(sid, rnd.randrange(3))
        else:
            sid = rnd.choice(live) if rnd.random() < 0.95 else -6
            if p.free(sid):
                live.remove(sid)
    for sid in list(live):
        assert p.free(sid)
    assert p.nat.num_free() == nb


def test_large_shared_prefix_pool_matches_the_oracle():
    """The long-context shape: eight requests behind one 4096-token prefix in
    a pool of a few thousand blocks, then a decode step's appends."""
    rng = np.random.default_rng(11)
    prefix = rng.integers(0, 32000, 4096).tolist()
    p = Pair(3000, 5)
    for s in range(8):
        tail = rng.integers(0, 32000, int(rng.integers(1, 3000))).tolist()
        assert p.add(s, prefix + tail)
    assert p.nat.add_sequence(100, prefix) == 4096
    p.ref.add_sequence(100, prefix)
    for _ in range(20):
        for s in range(8):
            assert p.append(s, int(rng.integers(0, 32000)))
    p.compare()


@pytest.mark.parametrize("call", [
    "create_blocks", "seq_id_add", "seq_id_append", "seq_id_free", "token", "token_array",
    "token_float", "max_blocks", "max_blocks_negative", "pad"])
def test_scalars_outside_the_c_types_are_refused_not_wrapped(call):
    # ctypes and numpy casts wrap silently; the binding refuses instead, and
    # the pool is left as it was
    status = 3 if call == "token_float" else 2
    pool = pkd.BlockPool(8)
    try:
        assert pool.add_sequence(1, list(range(20))) == 0
        before = pool.num_free()
        with pytest.raises(_lib.PaError) as e:
            if call == "create_blocks":
                pkd.BlockPool(2**32 + 4)
            elif call == "seq_id_add":
                pool.add_sequence(2**63, [1, 2, 3])
            elif call == "seq_id_append":
                pool.append_token(-2**63 - 1, 7)
            elif call == "seq_id_free":
                pool.free_sequence(2**64 + 1)
            elif call == "token":
                pool.append_token(1, 2**31)
            elif call == "token_array":
                pool.add_sequence(2, np.array([1, 2**32 + 1], dtype=np.int64))
            elif call == "token_float":
                pool.add_sequence(2, np.array([1.5, 2.0]))
            elif call == "max_blocks":
                pool.block_table([1], 2**32 + 2)
            elif call == "max_blocks_negative":
                pool.block_table([1], -1)
            elif call == "pad":
                pool.block_table([1], 4, pad=2**31)
        assert e.value.status == status, str(e.value)
        assert pool.num_free() == before
        table, lens = pool.block_table([1], 4)
        assert lens.tolist() == [20]
    finally:
        pool.close()
