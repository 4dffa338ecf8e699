"""Parity of the HIP path (through the C ABI) with the float64 oracle, plus the
invariants and edge cases of the method, on an MI355X.

Bar, against the oracle on the same stored (and, for fp8, dequantized) values:
every case meets the stated contract -- q/out in f32, f16 or bf16: max-abs <=
1e-2 and mean-abs <= 1e-3; fp8-e4m3 cache: max-abs <= 3e-2 -- and the tighter
of that and a bar set by the arithmetic of the io type. P is rounded to the io
type for the PV product (the running sum adds the same rounded values) and the
output once more at the end, so with unit roundoff u and |v| <= about 4.5 for
N(0,1) data the error is at most about u * (4.5 + 1): f32 (nothing rounded but
fp32 sums) max-abs 1e-5, mean 1e-6; f16 (u = 2^-11, 2.7e-3) 4e-3, 3e-4; bf16
(u = 2^-8, 2.1e-2) 2.5e-2, 1.5e-3. An fp8 cache widens exactly, so it takes
its io type's bar. The largest errors seen on MI355X are 6.7e-7 (f32), 1.0e-3
(f16), 9.4e-3 (bf16, contexts of a few tokens) and 1.4e-2 (bf16 q, fp8 cache,
two new tokens per sequence).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from tests.gpu_util import errors, to_device, to_f64

pytestmark = pytest.mark.gpu

TOL = {"max": 1e-2, "mean": 1e-3}          # the contract for f32/f16/bf16 caches
TOL_FP8 = {"max": 3e-2, "mean": 3e-3}      # the contract for an fp8 cache (mean reported)
# the io type's arithmetic (module docstring); each is within the contract
TIGHT = {"f32": {"max": 1e-5, "mean": 1e-6}, "f16": {"max": 4e-3, "mean": 3e-4},
         "bf16": {"max": 2.5e-2, "mean": 1.5e-3}}


def tol(spec):
    """The tighter of the contract and the io type's bar."""
    c = TOL_FP8 if spec.kv_dtype == "fp8_e4m3" else TOL
    t = TIGHT[spec.io_dtype]
    return {"max": min(c["max"], t["max"]), "mean": min(c["mean"], t["mean"])}


def run(wl, t=None, partition_size=None, lse=False, workspace=None, stream=None):
    t = t or to_device(wl)
    ps = wl.spec.partition_size if partition_size is None else partition_size
    B, Hq = wl.q.shape[:2]
    lse_out = torch.full((B, Hq), float("nan"), device="cuda") if lse else None
    out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                     float(wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                     partition_size=ps, workspace=workspace, lse_out=lse_out, stream=stream)
    torch.cuda.synchronize()
    return (out, lse_out) if lse else out


def ref(wl, seqs=None, lse=False):
    return oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                   wl.context_lens, wl.scale, wl.spec.io_dtype,
                                   wl.spec.kv_dtype, wl.k_scale, wl.v_scale,
                                   return_lse=lse, seqs=seqs)


def check(wl, got, expect, seqs=None, label=""):
    sel = slice(None) if seqs is None else list(seqs)
    g, r = got[sel], expect[sel]
    assert np.isfinite(g).all(), f"{label}: non-finite output"
    mx, mean = errors(g, r)
    print(f"  {label or wl.spec.name}: max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)
    t = tol(wl.spec)
    assert mx <= t["max"] and mean <= t["mean"], (label, mx, mean)
    return mx, mean


def small(k, batch, lens, **kw):
    return W.small_variant(W.SPECS[k], batch, lens, **kw)


SMALL = {
    "w1_tiny_f32": lambda: W.SPECS[1],
    "w2_f16_single_pass": lambda: small(2, 6, ("uniform", 16, 300)),
    "w3_f16_split512": lambda: small(3, 6, ("uniform", 100, 1400)),
    "w4_fp8kv_split512": lambda: small(4, 6, ("uniform", 100, 1400)),
    "w5_bf16_prefix_split512": lambda: small(5, 5, ("loguniform", 20, 6000)),
}


# ------------------------------------------------------------ small parity

@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity_with_lse(name):
    spec = SMALL[name]()
    print(f"case {name} {spec}", flush=True)
    wl = W.make_workload(spec)
    out, lse = run(wl, lse=True)
    exp_out, exp_lse = ref(wl, lse=True)
    check(wl, to_f64(out), exp_out, label=name)
    lerr = np.abs(lse.cpu().double().numpy() - exp_lse).max()
    print(f"  lse max-abs {lerr:.3e}", flush=True)
    assert lerr <= 5e-3


def test_golden_fixture():
    from tests.test_golden import load_golden
    spec, gout, glse = load_golden()
    wl = W.make_workload(spec)
    out, lse = run(wl, lse=True)
    check(wl, to_f64(out), gout, label="golden")
    assert np.abs(lse.cpu().double().numpy() - glse).max() <= 5e-3


@pytest.mark.parametrize("io,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                   ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3")])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ps", [0, 512])
def test_dtype_headdim_matrix(io, kv, D, ps):
    spec = W.Spec(f"mat_{io}_{kv}_d{D}_ps{ps}", 5, 12, 3, D, io, kv,
                  ("fixed", [1, 15, 16, 513, 1300]), 82, ("ratio", 1.2), ps, 0, D + ps)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    check(wl, to_f64(run(wl)), ref(wl), label=spec.name)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (32, 2), (9, 3), (5, 1), (16, 1)])
def test_group_sizes(hq, hkv):
    spec = W.Spec(f"grp_{hq}_{hkv}", 4, hq, hkv, 128, "f16", "f16",
                  ("fixed", [40, 600, 1030, 7]), 65, ("ratio", 1.2), 512, 0, hq * 100 + hkv)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    check(wl, to_f64(run(wl)), ref(wl), label=spec.name)


@pytest.mark.parametrize("ps", [16, 48, 64, 1024, 4096])
def test_partition_sizes(ps):
    spec = small(3, 4, ("fixed", [17, 300, 1000, 2100]), max_blocks_per_seq=140)
    wl = W.make_workload(spec)
    print(f"case partition {ps}", flush=True)
    check(wl, to_f64(run(wl, partition_size=ps)), ref(wl), label=f"ps{ps}")


@pytest.mark.parametrize("io,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                   ("f16", "fp8_e4m3")])
def test_two_level_merge(io, kv):
    """More than 16 partitions per sequence: groups of F partitions merge
    first, then the groups (140 partitions of 16 tokens at most here, so
    F = 16 and up to 9 groups). The lengths give eight full groups and a
    partial one (2240 tokens), a group of a single partition (257: 17
    partitions), exactly one level (256: 16 partitions), four groups (1000)
    and a short sequence."""
    spec = W.Spec(f"tree_{io}_{kv}", 5, 8, 2, 128, io, kv, ("fixed", [2240, 257, 256, 1000, 33]),
                  140, ("ratio", 1.2), 16, 0, 41)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    t = to_device(wl)
    out, lse = run(wl, t, lse=True)
    exp_out, exp_lse = ref(wl, lse=True)
    got = to_f64(out)
    check(wl, got, exp_out, label=spec.name)
    lerr = np.abs(lse.cpu().double().numpy() - exp_lse).max()
    print(f"  lse max-abs {lerr:.3e}", flush=True)
    assert lerr <= 5e-3
    # a second call on the same workspace finds the counters of both levels zero
    ws = torch.zeros(pkd.workspace_bytes(t["q"], t["k_cache"], t["block_table"], 16),
                     dtype=torch.uint8, device="cuda")
    a = to_f64(run(wl, t, partition_size=16, workspace=ws))
    b = to_f64(run(wl, t, partition_size=16, workspace=ws))
    assert np.array_equal(a, b) and np.array_equal(a, got)
    counters = ws[: 4 * 5 * 2 * (1 + 9)].view(torch.int32)
    assert int(counters.abs().sum()) == 0


# ------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("ps", [512, pkd.SPLIT_BALANCED])
def test_full_size_qwen2_5_1_5b_shape_in_the_split_modes_bench_times(ps):
    # The Qwen2.5-1.5B-shaped workload is specified as one pass, but bench.py
    # also times (and may report) 512-token partitions and the balanced split.
    spec = W.SPECS[2]
    print(f"case full workload 2 with partition_size {ps}", flush=True)
    wl = W.make_workload(spec)
    out = to_f64(run(wl, partition_size=ps))
    check(wl, out, ref(wl), label=f"full2 ps={ps}")




@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_full_size_workload(k):
    spec = W.SPECS[k]
    print(f"case full workload {k}: {spec.name}", flush=True)
    wl = W.make_workload(spec)
    out = to_f64(run(wl))
    assert np.isfinite(out).all()
    check(wl, out, ref(wl), label=f"full{k}")


# ------------------------------------------------------------- invariants

def test_block_permutation_is_bit_exact():
    spec = small(3, 6, ("uniform", 100, 1400))
    wl = W.make_workload(spec)
    a = run(wl).cpu()
    pi = np.random.default_rng(7).permutation(wl.num_blocks)
    wl2 = W.make_workload(spec)
    wl2.k_cache = np.empty_like(wl.k_cache)
    wl2.v_cache = np.empty_like(wl.v_cache)
    wl2.k_cache[pi] = wl.k_cache
    wl2.v_cache[pi] = wl.v_cache
    wl2.block_table = pi[wl.block_table].astype(np.int32)
    b = run(wl2).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("io,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                   ("f16", "fp8_e4m3")])
def test_one_token_context_returns_v(io, kv):
    spec = W.Spec(f"one_{io}_{kv}", 3, 8, 2, 128, io, kv, ("fixed", [1, 1, 1]), 4,
                  ("fixed", 12), 512, 0, 3)
    wl = W.make_workload(spec)
    got = to_f64(run(wl))
    expect = ref(wl)
    if kv == io:
        assert np.array_equal(got, expect)       # p = 1, sum = 1: exact
    else:
        check(wl, got, expect, label="one-token fp8")


def test_identical_v_rows_return_that_row():
    spec = small(3, 4, ("fixed", [33, 517, 1200, 2000]), max_blocks_per_seq=125)
    wl = W.make_workload(spec, poison=False)
    row = np.random.default_rng(1).standard_normal(128).astype(np.float16)
    wl.v_cache[:] = row.view(np.uint16)[None, None, :, None]
    got = to_f64(run(wl))
    want = np.broadcast_to(row.astype(np.float64), got.shape)
    assert np.abs(got - want).max() <= 1e-3 * np.abs(row).max()


def test_split_matches_single_pass():
    spec = small(3, 6, ("uniform", 100, 3000))
    wl = W.make_workload(spec)
    a, b = to_f64(run(wl, partition_size=0)), to_f64(run(wl, partition_size=512))
    assert np.abs(a - b).max() <= 1e-2


def test_run_to_run_bit_determinism():
    spec = small(5, 5, ("loguniform", 20, 20000))
    wl = W.make_workload(spec)
    t = to_device(wl)
    a = run(wl, t).cpu()
    b = run(wl, t).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_peaked_softmax():
    spec = small(3, 5, ("uniform", 200, 3000))
    wl = W.make_workload(spec)
    q = wl.q.view(np.float16).astype(np.float32) * 16
    wl.q = q.astype(np.float16).view(np.uint16)
    check(wl, to_f64(run(wl)), ref(wl), label="peaked q*16")


def test_rising_scores_rescale_every_page():
    # Scores rise monotonically along the context, so the running max moves
    # on every page.
    spec = W.Spec("ramp", 2, 4, 1, 128, "f32", "f32", ("fixed", [700, 1500]), 94,
                  ("ratio", 1.2), 512, 0, 8)
    wl = W.make_workload(spec)
    qv = wl.q[:, :, :].copy()
    u = np.zeros(128, dtype=np.float32)
    u[0] = 1.0
    wl.q[:] = np.float32(8.0) * u
    for b in range(2):
        L = int(wl.context_lens[b])
        for t in range(L):
            blk, slot = int(wl.block_table[b, t // 16]), t % 16
            wl.k_cache[blk, 0, 0, slot, 0] = np.float32(t / 40.0)
    del qv
    check(wl, to_f64(run(wl)), ref(wl), label="ramp")


def test_empty_contexts():
    spec = W.Spec("empty", 4, 8, 2, 128, "f16", "f16", ("fixed", [0, 5, 0, 700]), 44,
                  ("ratio", 1.2), 512, 0, 12)
    wl = W.make_workload(spec)
    out, lse = run(wl, lse=True)
    got = to_f64(out)
    assert np.array_equal(got[0], np.zeros_like(got[0])) and np.array_equal(got[2], got[0])
    l = lse.cpu().numpy()
    assert np.all(np.isneginf(l[0])) and np.all(np.isneginf(l[2]))
    check(wl, got, ref(wl), seqs=[1, 3], label="empty-mixed")


def test_workspace_reused_across_calls_and_streams():
    spec = small(3, 6, ("uniform", 100, 3000))
    wl1 = W.make_workload(spec)
    wl2 = W.make_workload(small(3, 6, ("uniform", 600, 2000)), seed=99)
    t1 = to_device(wl1)
    need = pkd.workspace_bytes(t1["q"], t1["k_cache"], t1["block_table"], 512)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    pkd.reset_workspace(ws)
    side = torch.cuda.Stream()
    for i in range(3):
        for wl in (wl1, wl2):
            with torch.cuda.stream(side):
                out = run(wl, partition_size=512, workspace=ws, stream=side)
            check(wl, to_f64(out), ref(wl), label=f"reuse{i}")


def test_nan_poison_never_leaks():
    # every parity workload carries NaN in its spare block and unread tail
    # slots; this case makes the tails as ragged as possible
    spec = W.Spec("poison", 6, 8, 2, 128, "bf16", "bf16", ("fixed", [1, 2, 15, 17, 31, 513]),
                  33, ("ratio", 1.2), 512, 0, 77)
    wl = W.make_workload(spec)
    got = to_f64(run(wl))
    assert np.isfinite(got).all()
    check(wl, got, ref(wl), label="poison")


def test_out_of_contract_metadata_gives_nan_not_a_fault():
    # Host-invisible metadata errors: one length beyond the table, one block
    # id beyond the pool. The kernel checks both before any cache access.
    spec = W.Spec("badmeta", 3, 8, 2, 128, "f16", "f16", ("fixed", [100, 200, 300]), 20,
                  ("ratio", 1.2), 512, 0, 5)
    wl = W.make_workload(spec)
    t = to_device(wl)
    t["context_lens"][0] = 20 * 16 + 1
    t["block_table"][1, 3] = wl.num_blocks + 1000
    got = to_f64(run(wl, t))
    assert np.isnan(got[0]).all() and np.isnan(got[1]).all()
    check(wl, got, ref(wl), seqs=[2], label="badmeta-ok-seq")


@pytest.mark.parametrize("io,kv", [("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8_e4m3"),
                                   ("f32", "f32")])
@pytest.mark.parametrize("ps", [0, 8192])
def test_long_units_cross_block_id_chunks(io, kv, ps):
    # A wave reads block ids 64 pages at a time; units of up to 9000 tokens
    # give each wave up to 141 pages, so the chunk refresh runs while K and V
    # loads for neighbouring pages are in flight.
    spec = W.Spec(f"long_{io}_{kv}_ps{ps}", 4, 8, 2, 128, io, kv,
                  ("fixed", [9000, 4097, 4096, 6100]), 563, ("ratio", 1.2), ps, 0, 31)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    check(wl, to_f64(run(wl)), ref(wl), label=spec.name)
