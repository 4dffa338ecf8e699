"""The balanced split's work line, checked on the host through the same header
the kernel compiles (tests/probes exports a host-side walk of every share).

Properties that must hold for any lengths: every page of every (sequence, KV
head) pair is read by exactly one piece; the pieces of a pair are numbered
0 .. nparts-1 in page order and sit in consecutive shares; workspace slots are
unique and below shares + B * H; shares differ by at most one page.
"""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = os.path.join(ROOT, "tests", "probes", "libpaprobes.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(PROBES):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(PROBES)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.pa_probe_schedule.argtypes = [ip, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ip, ctypes.c_int]
    lib.pa_probe_schedule.restype = ctypes.c_int
    return lib


def walk(lib, lens, H, mbs, shares):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int)
    n = lib.pa_probe_schedule(lens.ctypes.data_as(ip), len(lens), H, mbs, shares, None, 0)
    assert n > 0
    rows = np.zeros((n, 8), dtype=np.int32)
    m = lib.pa_probe_schedule(lens.ctypes.data_as(ip), len(lens), H, mbs, shares,
                              rows.ctypes.data_as(ip), n)
    assert m == n
    return rows


def pages(L, mbs):
    return 1 if (L <= 0 or L > 16 * mbs) else (L + 15) // 16


def check(lib, lens, H, mbs, shares):
    rows = walk(lib, lens, H, mbs, shares)
    B = len(lens)
    total = sum(pages(int(L), mbs) for L in lens) * H
    used = max(1, min(shares, total // 8))
    wg, b, g, lo, hi, k, nparts, slot0 = rows.T
    # shares come in order and differ by at most one page; a short line uses
    # fewer shares of at least 8 pages
    per_share = np.bincount(wg, weights=hi - lo).astype(np.int64)
    assert np.array_equal(np.unique(wg), np.arange(used))
    assert per_share.sum() == total and per_share.max() - per_share.min() <= 1
    assert used == 1 or per_share.min() >= 8
    # every pair covered exactly once, pieces in page order
    seen = set()
    for bb in range(B):
        for gg in range(H):
            sel = (b == bb) & (g == gg)
            assert sel.any(), (bb, gg)
            p = rows[sel]
            p = p[np.argsort(p[:, 5])]
            n = int(p[0, 6])
            assert len(p) == n and np.array_equal(p[:, 5], np.arange(n))
            assert (p[:, 6] == n).all() and (p[:, 7] == p[0, 7]).all()
            assert p[0, 3] == 0 and p[-1, 4] == pages(int(lens[bb]), mbs)
            assert np.array_equal(p[1:, 3], p[:-1, 4]) and (p[:, 4] > p[:, 3]).all()
            assert np.array_equal(np.diff(p[:, 0]), np.ones(n - 1))   # consecutive shares
            for kk in range(n):
                seen.add(int(p[0, 7]) + kk)
    slots = slot0 + k
    assert len(seen) == len(rows) == len(set(slots.tolist()))
    assert slots.min() >= 0 and slots.max() < shares + B * H
    return rows


@pytest.mark.parametrize("seed", range(12))
def test_random_lengths(lib, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 70))
    mbs = int(rng.integers(1, 300))
    lens = rng.integers(0, 16 * mbs + 1, size=B)
    lens[rng.random(B) < 0.1] = 0
    H = int(rng.choice([1, 2, 4, 8]))
    shares = int(rng.choice([1, 3, 7, 64, 768]))
    check(lib, lens, H, mbs, shares)


def test_out_of_contract_lengths_take_one_position(lib):
    rows = check(lib, np.array([-5, 0, 10_000, 33, 1 << 30]), 2, 100, 5)
    for bb in (0, 1, 2, 4):
        sel = rows[rows[:, 1] == bb]
        assert len(sel) == 2 and (sel[:, 4] - sel[:, 3] == 1).all()


def test_one_long_sequence_spans_many_shares(lib):
    rows = check(lib, np.array([131072]), 8, 8192, 768)
    assert rows[:, 6].max() >= 90


def test_many_short_sequences_share_one_workgroup(lib):
    rows = check(lib, np.ones(4096, dtype=np.int64), 1, 4, 768)
    assert (rows[:, 6] == 1).all()                 # nothing to merge
    assert np.bincount(rows[:, 0]).max() == 8      # the minimum share


def test_headline_shape(lib):
    rng = np.random.default_rng(3)
    lens = rng.integers(512, 4097, size=32)
    rows = check(lib, lens, 4, 256, 768)
    assert rows[:, 0].max() == 767       # every workgroup gets a share


def test_floor_div_is_exact_integer_division(lib):
    """The work line divides through doubles (pa_schedule.h floor_div); it must
    equal integer division on the whole range the schedule uses: quotients
    just below an integer (a = k*b - 1), the largest products of a share
    index and a line length, and divisors up to 2^31 - 1."""
    lib.pa_probe_floor_div.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.pa_probe_floor_div.restype = None
    rng = np.random.default_rng(5)
    a, b = [], []
    for _ in range(20000):
        bb = int(rng.integers(1, 2**31))
        k = int(rng.integers(0, min(2**31 - 1, (2**46) // bb) + 1))
        for aa in (k * bb - 1, k * bb, k * bb + 1, k * bb + bb - 1):
            if 0 <= aa < 2**46 and aa // bb < 2**31:
                a.append(aa)
                b.append(bb)
    # share starts and share lookups at the largest sizes the kernel accepts
    for s in (1, 255, 256, 257, 768, 12288):
        for n in (1, 8, 2**31 - 1, 2**31 - 12289, 123456789):
            for w in (0, 1, s // 2, s - 1, s):
                a.append(w * n); b.append(s)
            for x in (0, 1, n // 2, n - 1):
                a.append((x + 1) * s - 1); b.append(n)
    a = np.array(a, dtype=np.int64)
    b = np.array(b, dtype=np.int64)
    out = np.empty(len(a), dtype=np.int32)
    lib.pa_probe_floor_div(a.ctypes.data, b.ctypes.data, len(a), out.ctypes.data)
    np.testing.assert_array_equal(out.astype(np.int64), a // b)


def test_shares_numbered_xcd_by_xcd(lib):
    """Workgroup blk of the balanced kernel's grid takes share
    share_of_block(blk, grid, S): every share exactly once, neighbouring
    shares on the same XCD (workgroups go to the 8 XCDs in turn, so XCD =
    blk % 8) except at the boundaries between XCDs, and a short line spread
    over all 8 XCDs."""
    lib.pa_probe_share_of_block.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.pa_probe_share_of_block.restype = None
    for grid in (8, 16, 248, 256, 768, 1024, 7, 255):
        for S in sorted({1, 2, 7, 8, 9, 40, 63, 64, 65, grid // 2, grid - 1, grid} - {0}):
            if S > grid:
                continue
            out = np.empty(grid, dtype=np.int32)
            lib.pa_probe_share_of_block(grid, S, out.ctypes.data)
            taken = out[out < S]
            assert sorted(taken.tolist()) == list(range(S)), (grid, S)
            assert (out <= S).all()
            if grid % 8:
                assert (out[:S] == np.arange(S)).all()
                continue
            xcd = np.empty(S, dtype=np.int64)
            xcd[taken] = np.nonzero(out < S)[0] % 8
            per = -(-S // 8)
            # consecutive shares share an XCD except every per-th boundary
            same = (xcd[1:] == xcd[:-1]).sum()
            assert same >= S - 1 - 7, (grid, S, same)
            assert len(set(xcd.tolist())) == min(8, -(-S // per)), (grid, S)
