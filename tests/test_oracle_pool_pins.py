"""Pins for the block-pool oracle (oracle/block_pool.py): FNV-1a-64 test
vectors from its published definition, a hand-worked scenario of prefix
reuse, eviction and capacity failures, shared-prefix tables like the
long-context workload's, and invariants over random operation sequences.
CPU only."""
import random

import pytest

from oracle import BlockPoolRef, PoolError, chain_hash, fnv1a64


def test_fnv1a64_published_vectors():
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_chained_hash_depends_on_parent_and_tokens():
    t = list(range(16))
    assert chain_hash(1, t) != chain_hash(2, t)
    assert chain_hash(1, t) != chain_hash(1, t[:15] + [99])
    assert chain_hash(1, t) == chain_hash(1, list(t))


def test_hand_worked_scenario():
    p = BlockPoolRef(6, seed=7)
    A = list(range(40))
    assert p.add_sequence("A", A) == 0
    assert p.seqs["A"]["blocks"] == [0, 1, 2]
    B = list(range(32)) + list(range(100, 110))
    assert p.add_sequence("B", B) == 32                  # two full blocks shared
    assert p.seqs["B"]["blocks"] == [0, 1, 3] and p.ref[:4] == [2, 2, 1, 1]
    p.free_sequence("A")                                  # releases 2, keeps 0 and 1 for B
    assert list(p.free) == [4, 5, 2]
    assert p.add_sequence("C", list(range(500, 532))) == 0
    assert p.seqs["C"]["blocks"] == [4, 5] and list(p.free) == [2]
    for tok in range(110, 116):                           # B's third block fills up
        p.append_token("B", tok)
    assert p.seqs["B"]["blocks"] == [0, 1, 3]
    h2 = chain_hash(p.key[1][0], list(range(100, 116)))
    assert p.cached[h2] == 3
    p.append_token("B", 116)                              # a fourth block: the free one
    assert p.seqs["B"]["blocks"] == [0, 1, 3, 2] and p.num_free() == 0
    D = list(range(16)) + [1, 2, 3]
    with pytest.raises(PoolError):                        # no block for D's partial block
        p.add_sequence("D", D)
    assert "D" not in p.seqs and p.ref[0] == 1
    p.free_sequence("C")                                  # releases 5, then 4
    assert list(p.free) == [5, 4]
    assert p.add_sequence("D", D) == 16
    assert p.seqs["D"]["blocks"] == [0, 5]                # 5 evicted (C's second block)
    with pytest.raises(PoolError):                        # C's first block still cached (4),
        p.add_sequence("E", list(range(500, 532)))        # its second was evicted: needs 2, has 1
    assert list(p.free) == [4]


def test_shared_prefix_tables_like_the_long_context_workload():
    prefix = [7] * 4096
    p = BlockPoolRef(2000, seed=1)
    for s in range(8):
        tail = [1000 + s] * (100 + 37 * s)
        got = p.add_sequence(s, prefix + tail)
        assert got == (0 if s == 0 else 4096)
    rows, lens = p.block_table(list(range(8)), 300, -1)
    for s in range(1, 8):
        assert rows[s][:256] == rows[0][:256]
        assert len(set(rows[s][256:]) & set(rows[0][256:]) - {-1}) == 0
    assert lens == [4096 + 100 + 37 * s for s in range(8)]


def check_invariants(p):
    held = {}
    for s in p.seqs.values():
        assert len(s["blocks"]) == -(-len(s["tokens"]) // 16)
        assert len(set(s["blocks"])) == len(s["blocks"])
        for b in s["blocks"]:
            held[b] = held.get(b, 0) + 1
    for b in range(p.n):
        assert p.ref[b] == held.get(b, 0)
        assert (b in p.free) == (p.ref[b] == 0)
    for h, b in p.cached.items():
        assert p.key[b] is not None and p.key[b][0] == h
        assert chain_hash(p.key[b][1], list(p.key[b][2])) == h


@pytest.mark.parametrize("seed", range(6))
def test_invariants_over_random_operations(seed):
    rng = random.Random(seed)
    p = BlockPoolRef(rng.choice([8, 40, 200]), seed=seed)
    prompts = [[rng.randrange(5) for _ in range(rng.randrange(0, 90))] for _ in range(6)]
    live, nid = [], 0
    for _ in range(400):
        op = rng.random()
        try:
            if op < 0.35:
                base = rng.choice(prompts)
                toks = base[: rng.randrange(len(base) + 1)] + [rng.randrange(5) for _ in range(rng.randrange(20))]
                p.add_sequence(nid, toks)
                live.append(nid)
                nid += 1
            elif op < 0.8 and live:
                p.append_token(rng.choice(live), rng.randrange(5))
            elif live:
                sid = live.pop(rng.randrange(len(live)))
                p.free_sequence(sid)
        except PoolError:
            pass
        check_invariants(p)
