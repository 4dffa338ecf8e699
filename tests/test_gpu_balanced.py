"""The balanced split (partition_size = SPLIT_BALANCED) against the float64
oracle, through the C ABI, on an MI355X.

The balanced split cuts the pages of all (sequence, KV head) pairs into equal
shares, one per resident workgroup, and merges a pair's pieces by log-sum-exp,
so its output must meet the same bar as the other modes: max-abs <= 1e-2 and
mean-abs <= 1e-3 for f32/f16/bf16 caches, max-abs <= 3e-2 for fp8-e4m3.
The cases stress what is new in it: the workgroup-wide scan of the lengths
(batch 1 .. 4096, ragged per-thread chunks), shares that hold many short
sequences, pairs cut into many pieces, and empty or out-of-contract sequences
that occupy one placeholder position of the work line.
"""
import numpy as np
import pytest
import torch

import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from tests.gpu_util import to_device, to_f64
from tests.test_gpu_parity import SMALL, check, ref, run

pytestmark = pytest.mark.gpu

BAL = pkd.SPLIT_BALANCED


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workloads(name):
    spec = SMALL[name]()
    print(f"case balanced {name}", flush=True)
    wl = W.make_workload(spec)
    out, lse = run(wl, partition_size=BAL, lse=True)
    exp_out, exp_lse = ref(wl, lse=True)
    check(wl, to_f64(out), exp_out, label=f"bal {name}")
    lerr = np.abs(lse.cpu().double().numpy() - exp_lse).max()
    print(f"  lse max-abs {lerr:.3e}", flush=True)
    assert lerr <= 5e-3


@pytest.mark.parametrize("io,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                   ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3")])
@pytest.mark.parametrize("D", [64, 128])
def test_dtype_headdim_matrix(io, kv, D):
    spec = W.Spec(f"bal_{io}_{kv}_d{D}", 5, 12, 3, D, io, kv,
                  ("fixed", [1, 15, 16, 513, 1300]), 82, ("ratio", 1.2), BAL, 0, D + 7)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    check(wl, to_f64(run(wl)), ref(wl), label=spec.name)


@pytest.mark.parametrize("batch,lens,hkv", [
    (1, ("fixed", [60000]), 8),              # one pair cut into ~90 pieces
    (300, ("uniform", 1, 700), 2),           # two sequences per scan thread, ragged
    (4096, ("uniform", 0, 40), 1),           # largest batch: 16 per thread, tiny shares
    (257, ("uniform", 1, 3000), 4),          # one sequence past a thread's chunk
])
def test_batch_and_length_extremes(batch, lens, hkv):
    top = max(lens[1]) if lens[0] == "fixed" else lens[2]
    spec = W.Spec(f"bal_b{batch}_hkv{hkv}", batch, 2 * hkv, hkv, 128, "bf16", "bf16", lens,
                  max(1, -(-top // 16)), ("ratio", 1.2), BAL, 0, batch + hkv)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    check(wl, to_f64(run(wl)), ref(wl), label=spec.name)


@pytest.mark.parametrize("k", [3, 4, 5])
def test_full_size_workload(k):
    spec = W.SPECS[k]
    print(f"case balanced full workload {k}: {spec.name}", flush=True)
    wl = W.make_workload(spec)
    out = to_f64(run(wl, partition_size=BAL))
    check(wl, out, ref(wl), label=f"bal full{k}")


def test_matches_fixed_partitions_and_is_deterministic():
    spec = W.small_variant(W.SPECS[5], 6, ("loguniform", 20, 30000))
    wl = W.make_workload(spec)
    t = to_device(wl)
    a = run(wl, t, partition_size=BAL).cpu()
    b = run(wl, t, partition_size=BAL).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    c = run(wl, t, partition_size=512).cpu()
    assert np.abs(to_f64(a) - to_f64(c)).max() <= 1e-2


def test_empty_and_out_of_contract_sequences():
    spec = W.Spec("bal_edge", 6, 8, 2, 128, "f16", "f16", ("fixed", [0, 5, 0, 700, 300, 2000]),
                  130, ("ratio", 1.2), BAL, 0, 21)
    wl = W.make_workload(spec)
    t = to_device(wl)
    t["context_lens"][4] = 130 * 16 + 1           # length beyond the table
    t["block_table"][5, 40] = wl.num_blocks + 7    # block id beyond the pool
    B, Hq = wl.q.shape[:2]
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                     float(wl.scale), partition_size=BAL, lse_out=lse)
    torch.cuda.synchronize()
    got = to_f64(out)
    l = lse.cpu().numpy()
    assert np.array_equal(got[0], np.zeros_like(got[0])) and np.array_equal(got[2], got[0])
    assert np.all(np.isneginf(l[0])) and np.all(np.isneginf(l[2]))
    assert np.isnan(got[4]).all() and np.isnan(got[5]).all()
    check(wl, got, ref(wl), seqs=[1, 3], label="bal edge")


def test_workspace_reused_across_shapes():
    wls = [W.make_workload(W.small_variant(W.SPECS[3], 6, ("uniform", 100, 3000))),
           W.make_workload(W.small_variant(W.SPECS[3], 6, ("uniform", 600, 2000)), seed=99),
           W.make_workload(W.small_variant(W.SPECS[3], 6, ("uniform", 1, 200)), seed=5)]
    t0 = to_device(wls[0])
    need = pkd.workspace_bytes(t0["q"], t0["k_cache"], t0["block_table"], BAL)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    pkd.reset_workspace(ws)
    for i in range(2):
        for wl in wls:
            out = run(wl, partition_size=BAL, workspace=ws)
            check(wl, to_f64(out), ref(wl), label=f"bal reuse{i}")


@pytest.mark.parametrize("ps", [512, BAL])
def test_workspace_serves_smaller_calls_without_reset(ps):
    # The counters sit at the start of the workspace, so after a call with
    # more (sequence, KV head) pairs a call with fewer (and another table
    # width) finds its counters zero without a reset.
    big = W.make_workload(W.small_variant(W.SPECS[3], 8, ("uniform", 100, 3000)))
    small = W.make_workload(W.small_variant(W.SPECS[3], 3, ("uniform", 600, 2000)), seed=98)
    tb = to_device(big)
    need = pkd.workspace_bytes(tb["q"], tb["k_cache"], tb["block_table"], ps)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    pkd.reset_workspace(ws)
    for i in range(2):
        for wl in (big, small, small):
            out = run(wl, partition_size=ps, workspace=ws)
            check(wl, to_f64(out), ref(wl), label=f"ws order {i} {wl.spec.batch}")


@pytest.mark.parametrize("ps", [512, BAL])
def test_workspace_rule_big_small_big_across_a_counter_boundary(ps):
    # B=32 with 4 KV heads (512 counter bytes), then 2 KV heads (256 bytes),
    # then 4 again: the small call's partial results cover the big call's
    # counters 64..127, so the header's rule asks for a reset before the
    # third call (its counter bytes exceed the smallest since the last reset)
    big = W.make_workload(W.small_variant(W.SPECS[3], 32, ("uniform", 100, 1500)))
    small = W.make_workload(W.small_variant(W.SPECS[2], 32, ("uniform", 100, 1500)), seed=77)
    need = max(pkd.workspace_bytes(to_device(w)["q"], to_device(w)["k_cache"],
                                   to_device(w)["block_table"], ps) for w in (big, small))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    pkd.reset_workspace(ws)
    for i, wl in enumerate((big, small, big)):
        if i == 2:
            pkd.reset_workspace(ws)
        print(f"case workspace rule ps={ps} call {i}: Hkv {wl.spec.num_kv_heads}", flush=True)
        out = run(wl, partition_size=ps, workspace=ws)
        check(wl, to_f64(out), ref(wl), label=f"rule {ps} call {i}")


def _stale_case(ps, counter_index, value, spec):
    wl = W.make_workload(spec)
    t = to_device(wl)
    need = pkd.workspace_bytes(t["q"], t["k_cache"], t["block_table"], ps)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ws.view(torch.int32)[counter_index] = value
    return wl, t, ws


@pytest.mark.parametrize("ps,counter,label", [
    (512, 0, "pair counter, one merge level"),
    (BAL, 0, "pair counter, balanced split"),
    (16, 2 * 2 + 0, "first merge-group counter of pair 0, two merge levels"),
    (16, 0, "pair counter, two merge levels")])
def test_stale_counter_gives_nan_rows_until_reset(ps, counter, label):
    # A counter left at or above the number of pieces it counts (a broken
    # reuse rule) makes the rows of its (sequence, KV head) NaN, every other
    # row stays right, the state persists, and a reset restores the call.
    spec = W.Spec("stale", 2, 8, 2, 128, "f16", "f16", ("fixed", [3000, 700]), 200,
                  ("ratio", 1.2), ps, 0, 5)
    print(f"case stale counter ps={ps}: {label}", flush=True)
    wl, t, ws = _stale_case(ps, counter, 1000, spec)
    exp = ref(wl)
    G = spec.num_q_heads // spec.num_kv_heads
    for rep in range(2):
        out = to_f64(run(wl, t, partition_size=ps, workspace=ws))
        assert np.isnan(out[0, :G]).all(), (label, rep)                # pair (0, 0)
        assert np.isfinite(out[0, G:]).all() and np.isfinite(out[1]).all()
        assert np.abs(out[0, G:] - exp[0, G:]).max() <= 1e-2
        assert np.abs(out[1] - exp[1]).max() <= 1e-2
    pkd.reset_workspace(ws)
    out = to_f64(run(wl, t, partition_size=ps, workspace=ws))
    check(wl, out, exp, label=f"stale {label} after reset")


def test_bit_identical_when_merging_workgroups_hold_several_pairs():
    # Short shares cut each pair into more than 8 pieces, and which workgroup
    # finishes a pair last (and so merges it, maybe together with other pairs)
    # changes from run to run; the merge's slicing depends on the pair alone,
    # so every run gives the same bits.
    spec = W.small_variant(W.SPECS[3], 8, ("uniform", 100, 3000))
    wl = W.make_workload(spec, seed=40)
    t = to_device(wl)
    first = run(wl, t, partition_size=BAL).cpu()
    for i in range(12):
        again = run(wl, t, partition_size=BAL).cpu()
        assert torch.equal(first.view(torch.int16), again.view(torch.int16)), i
    check(wl, to_f64(first), ref(wl), label="bal determinism")


def test_fp8_merges_of_more_pieces_than_one_batch_are_bit_identical():
    # With an fp8 cache a merge takes four pieces per batch: pairs cut into
    # about five to nine pieces here take two or more slices, combined in
    # order through LDS, whichever workgroup finishes the pair
    spec = W.small_variant(W.SPECS[4], 10, ("uniform", 1000, 3000))
    wl = W.make_workload(spec, seed=43)
    print(f"case fp8 slices {spec.name}", flush=True)
    t = to_device(wl)
    first = run(wl, t, partition_size=BAL).cpu()
    for i in range(8):
        again = run(wl, t, partition_size=BAL).cpu()
        assert torch.equal(first.view(torch.int16), again.view(torch.int16)), i
    check(wl, to_f64(first), ref(wl), label="bal fp8 slices")
