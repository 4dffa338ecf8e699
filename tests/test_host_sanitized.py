"""The library's host code built for the CPU alone under AddressSanitizer and
UndefinedBehaviorSanitizer (g++, no HIP, no GPU): the argument checks and
workspace layouts every entry point runs before a launch (csrc/pa_host.h,
the same header the library compiles), the balanced split's work line and
the shared-prefix schedule (csrc/pa_schedule.h) and the block pool
(csrc/block_pool.cpp).
tests/sanitize/host_checks.cpp holds the checks; here it is built and run,
and its block-pool results are compared with the oracle's pool on the
operation sequences the pool tests use. Any sanitizer report fails the test."""
import os
import random
import shutil
import subprocess

import numpy as np
import pytest

from oracle import BlockPoolRef, PoolError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_decode_05_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
           os.path.join(CSRC, "block_pool.cpp")]
EXE = os.path.join(ROOT, "_build", "host_checks_sanitized")
PA_ERR_SHAPE, PA_ERR_CAPACITY, PA_ERR_STATE = 2, 7, 8

SAN_ENV = dict(os.environ,
               ASAN_OPTIONS="halt_on_error=1:detect_stack_use_after_return=1:strict_string_checks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


@pytest.fixture(scope="module")
def exe():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not installed")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *SOURCES, "-o", EXE]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return EXE


def run(exe, *args, stdin=None):
    res = subprocess.run([exe, *map(str, args)], input=stdin, capture_output=True, text=True,
                         timeout=600, env=SAN_ENV)
    report = res.stderr
    assert res.returncode == 0 and "runtime error" not in report and "Sanitizer" not in report, \
        (res.returncode, res.stdout[-2000:], report[-4000:])
    assert "FAIL" not in res.stdout, res.stdout[-2000:]
    return res.stdout


def test_argument_checks_give_the_documented_statuses(exe):
    assert "args: ok" in run(exe, "args")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_layouts_of_random_shapes_around_every_limit(exe, seed):
    out = run(exe, "fuzz", 200000, seed)
    assert "fuzz:" in out and out.strip().endswith("ok")
    # a fair share of the draws must pass the checks, or the layouts go untested
    accepted = int(out.split(",")[1].split()[0])
    assert accepted > 2000, out


@pytest.mark.parametrize("seed", [1, 2])
def test_balanced_work_line_covers_every_page_once(exe, seed):
    assert run(exe, "line", 400, seed).strip().endswith("ok")


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_shared_prefix_schedule_covers_every_page_once(exe, seed):
    out = run(exe, "prefix", 300, seed)
    assert out.strip().endswith("ok"), out


class Script:
    """Block-pool operations for the sanitized driver, with the oracle's
    expected result line for each."""

    def __init__(self, num_blocks, seed):
        self.ref = BlockPoolRef(num_blocks, seed)
        self.ops = [f"C {num_blocks} {seed}"]
        self.want = ["C 0"]

    def _do(self, op, fn, ok_line, err):
        self.ops.append(op)
        try:
            r = fn()
        except PoolError as e:
            self.want.append(("err", op[0], err(str(e))))
            return False
        self.want.append(ok_line(r))
        return True

    def add(self, sid, toks):
        return self._do(f"A {sid} {len(toks)} " + " ".join(map(str, toks)),
                        lambda: self.ref.add_sequence(sid, toks), lambda r: f"A 0 {r}",
                        lambda m: PA_ERR_STATE if "exists" in m else PA_ERR_CAPACITY)

    def append(self, sid, tok):
        return self._do(f"P {sid} {tok}", lambda: self.ref.append_token(sid, tok), lambda r: "P 0",
                        lambda m: PA_ERR_STATE if "no such" in m else PA_ERR_CAPACITY)

    def free(self, sid):
        return self._do(f"F {sid}", lambda: self.ref.free_sequence(sid), lambda r: "F 0",
                        lambda m: PA_ERR_STATE)

    def snapshot(self, mbs=None, pad=-1):
        sids = sorted(self.ref.seqs)
        self.ops.append("N")
        self.want.append(f"N {self.ref.num_free()}")
        if sids:
            mbs = mbs or max(len(s["blocks"]) for s in self.ref.seqs.values()) + 1
            rows, lens = self.ref.block_table(sids, mbs, pad)
            self.ops.append(f"T {pad} {mbs} {len(sids)} " + " ".join(map(str, sids)))
            flat = [x for r in rows for x in r]
            self.want.append("T 0 " + " ".join(map(str, flat)) + " | " + " ".join(map(str, lens)))

    def shared(self, sids):
        """The shared prefix of sids, expected from the oracle's pool state
        by the definition (tests/test_pool.py)."""
        from tests.test_pool import expected_shared_prefix
        self.ops.append(f"S {len(sids)} " + " ".join(map(str, sids)))
        if all(sid in self.ref.seqs for sid in sids):
            self.want.append(f"S 0 {expected_shared_prefix(self.ref, list(sids))}")
        else:
            self.want.append(("err", "S", PA_ERR_STATE))

    def check(self, exe):
        out = run(exe, "pool", stdin="\n".join(self.ops + ["D"]) + "\n").splitlines()
        assert len(out) == len(self.want) + 1 and out[-1] == "D", out[-3:]
        for op, want, got in zip(self.ops, self.want, out):
            if isinstance(want, tuple):
                _, kind, status = want
                assert got.split()[:2] == [kind, str(status)], (op[:80], got)
            else:
                assert got.split() == want.split(), (op[:80], got[:200], want[:200])


def test_pool_hand_worked_and_error_scenarios(exe):
    s = Script(6, 7)
    assert s.add(1, list(range(40)))
    assert s.add(2, list(range(32)) + list(range(100, 110)))
    assert s.free(1)
    assert s.add(3, list(range(500, 532)))
    for tok in range(110, 117):
        assert s.append(2, tok)
    assert not s.add(4, list(range(16)) + [1, 2, 3])
    assert not s.add(2, [1])                       # exists
    assert not s.append(9, 1) and not s.free(9)    # unknown
    assert s.free(3)
    assert s.add(4, list(range(16)) + [1, 2, 3])
    assert s.add(10, [])
    s.snapshot()
    s.snapshot(pad=-7)
    s.check(exe)


@pytest.mark.parametrize("seed", range(4))
def test_pool_random_operation_sequences(exe, seed):
    """The random mix of the pool tests: prompts from a few shared prefixes,
    appends from a 3-token vocabulary, a pool small enough to run out and
    evict, and unknown ids."""
    rnd = random.Random(seed)
    nb = rnd.choice([12, 24, 40])
    s = Script(nb, seed * 7919)
    prefixes = [[rnd.randrange(50) for _ in range(rnd.choice([16, 32, 48, 20]))]
                for _ in range(3)]
    next_id, live = 0, []
    for i in range(600):
        r = rnd.random()
        if r < 0.3 or not live:
            toks = list(rnd.choice(prefixes)) if rnd.random() < 0.7 else []
            toks = toks[: rnd.randrange(len(toks) + 1)] if rnd.random() < 0.3 else toks
            toks += [rnd.randrange(3) for _ in range(rnd.randrange(0, 40))]
            sid = next_id if rnd.random() < 0.95 or not live else rnd.choice(live)
            if s.add(sid, toks):
                live.append(sid)
            next_id += sid == next_id
        elif r < 0.8:
            s.append(rnd.choice(live) if rnd.random() < 0.97 else -5, rnd.randrange(3))
        else:
            sid = rnd.choice(live) if rnd.random() < 0.95 else -6
            if s.free(sid):
                live.remove(sid)
        if i % 50 == 0:
            s.snapshot()
        if i % 25 == 0 and live:
            s.shared(rnd.sample(live, rnd.randint(1, len(live))) + ([10 ** 6] if i % 100 == 0 else []))
    for sid in list(live):
        assert s.free(sid)
    s.snapshot()
    s.check(exe)


def test_pool_long_shared_prefix(exe):
    rng = np.random.default_rng(11)
    prefix = rng.integers(0, 32000, 4096).tolist()
    s = Script(3000, 5)
    for q in range(8):
        assert s.add(q, prefix + rng.integers(0, 32000, int(rng.integers(1, 3000))).tolist())
    assert s.add(100, prefix)
    for _ in range(20):
        for q in range(8):
            assert s.append(q, int(rng.integers(0, 32000)))
    s.shared(list(range(8)))
    s.shared([100, 3, 5])
    s.snapshot()
    s.check(exe)
