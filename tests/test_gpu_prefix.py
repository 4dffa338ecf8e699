"""The shared-prefix decode (pa_decode_prefix) against the float64 oracle,
through the C ABI, on an MI355X.

The call computes the same decode as pa_decode: the oracle reads every
sequence's pages through its own block-table row, and the kernel reads the
declared shared pages once (from the row of a longest sequence) for all rows,
the rest per sequence, and merges both by log-sum-exp. So the bar is the one
of every other mode (tests/test_gpu_parity.py `tol`). The cases cover the
geometry of the prefix pass (16 / G sequences per tile, passes of one to four
tiles, a wave left idle with three), sequences shorter than the prefix (their
last prefix page partial, shared or private), declared prefixes shorter or
longer than the shared one, a broken declaration (NaN rows for exactly the
sequences it touches), empty and out-of-contract sequences, the workspace
shared with the plain balanced split, stale counters and determinism.
"""
import numpy as np
import pytest
import torch

import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from tests.gpu_util import to_device, to_f64
from tests.test_gpu_parity import check, ref, run

pytestmark = pytest.mark.gpu

BAL = pkd.SPLIT_BALANCED


def run_prefix(wl, P, t=None, lse=False, workspace=None):
    t = t or to_device(wl)
    B, Hq = wl.q.shape[:2]
    lse_out = torch.full((B, Hq), float("nan"), device="cuda") if lse else None
    out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                     float(wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"],
                     partition_size=BAL, workspace=workspace, lse_out=lse_out, prefix_blocks=P)
    torch.cuda.synchronize()
    return (out, lse_out) if lse else out


def spec(name, B, hq, hkv, D, io, kv, lens, prefix_tokens, seed, mbs=None):
    top = max(lens[1]) if lens[0] == "fixed" else lens[2]
    mbs = mbs or max(1, -(-max(top, prefix_tokens) // 16))
    return W.Spec(name, B, hq, hkv, D, io, kv, lens, mbs, ("ratio", 1.2), BAL, prefix_tokens, seed)


# (spec, declared prefix blocks): G, sequences per tile and passes vary; the
# lengths include sequences shorter than the prefix, at a page boundary, empty.
CASES = {
    "g4_b8_bf16_d128_short_and_long": (
        spec("p_g4", 8, 32, 8, 128, "bf16", "bf16",
             ("fixed", [5000, 4096, 4100, 1275, 16, 0, 17, 9000]), 4096, 11), 256),
    "g7_b9_f16_two_passes": (
        spec("p_g7", 9, 28, 4, 128, "f16", "f16", ("uniform", 1, 6000), 2048, 12), 128),
    "g16_b13_f32_d64_four_passes": (
        spec("p_g16", 13, 16, 1, 64, "f32", "f32", ("uniform", 300, 2500), 1024, 13), 64),
    "g1_b70_fp8_one_tile_last_pass": (
        spec("p_g1", 70, 4, 4, 128, "f16", "fp8_e4m3", ("uniform", 50, 1500), 512, 14), 32),
    "g2_b20_bf16_fp8_d64_three_tiles": (
        spec("p_g2", 20, 4, 2, 64, "bf16", "fp8_e4m3", ("uniform", 1, 3000), 800, 15), 50),
    "declared_shorter_than_shared": (
        spec("p_short", 6, 32, 8, 128, "bf16", "bf16", ("uniform", 2000, 7000), 4096, 16), 100),
    "declared_beyond_every_sequence": (
        spec("p_beyond", 5, 28, 4, 128, "f16", "f16", ("fixed", [300, 700, 33, 64, 640]), 1024, 17),
        64),
    "declared_zero": (
        spec("p_zero", 5, 28, 4, 128, "f16", "f16", ("uniform", 1, 3000), 1024, 18), 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_shared_prefix_parity_with_lse(name):
    sp, P = CASES[name]
    print(f"case prefix {name} P={P}", flush=True)
    wl = W.make_workload(sp)
    out, lse = run_prefix(wl, P, lse=True)
    exp_out, exp_lse = ref(wl, lse=True)
    got = to_f64(out)
    l = lse.cpu().double().numpy()
    live = [b for b in range(sp.batch) if wl.context_lens[b] > 0]
    for b in range(sp.batch):
        if wl.context_lens[b] == 0:
            assert np.array_equal(got[b], np.zeros_like(got[b])) and np.all(np.isneginf(l[b]))
    check(wl, got, exp_out, seqs=live, label=f"prefix {name}")
    lerr = np.abs(l[live] - exp_lse[live]).max()
    print(f"  lse max-abs {lerr:.3e}", flush=True)
    assert lerr <= 5e-3


def test_small_llama3_8b_shaped_shared_prefix():
    sp = W.small_variant(W.SPECS[5], 6, ("loguniform", 20, 30000))
    wl = W.make_workload(sp)
    print(f"case prefix {sp.name}", flush=True)
    check(wl, to_f64(run_prefix(wl, sp.shared_prefix_tokens // 16)), ref(wl), label=sp.name)


def test_full_size_llama3_8b_shared_prefix_workload():
    sp = W.SPECS[5]
    print(f"case prefix full {sp.name}", flush=True)
    wl = W.make_workload(sp)
    check(wl, to_f64(run_prefix(wl, sp.shared_prefix_tokens // 16)), ref(wl), label="prefix full5")


def _free_block(wl):
    used = set(int(x) for x in np.unique(wl.block_table)) | {wl.spare_block}
    return next(i for i in range(wl.num_blocks) if i not in used)


def test_private_partial_last_prefix_page():
    # A sequence that ends inside the prefix keeps its partial last page in a
    # block of its own (as a block pool that shares only full blocks does):
    # that page is part of its suffix, not of the shared prefix.
    sp = spec("p_priv", 5, 32, 8, 128, "bf16", "bf16", ("fixed", [4000, 1275, 3000, 2050, 900]),
              4096, 19)
    wl = W.make_workload(sp)
    for b in (1, 4):
        j = int(wl.context_lens[b]) // 16
        old, new = int(wl.block_table[b, j]), _free_block(wl)
        wl.k_cache[new] = wl.k_cache[old]
        wl.v_cache[new] = wl.v_cache[old]
        wl.block_table[b, j] = new
    check(wl, to_f64(run_prefix(wl, 256)), ref(wl), label="prefix private partial page")


def test_broken_declaration_gives_nan_rows_of_exactly_those_sequences():
    sp = spec("p_broken", 6, 32, 8, 128, "f16", "f16", ("fixed", [3000, 5000, 900, 4000, 4096, 100]),
              4096, 20)
    wl = W.make_workload(sp)
    exp = ref(wl)
    # sequence 3 points one of its shared pages elsewhere (a page of sequence
    # 1's suffix)
    wl.block_table[3, 10] = wl.block_table[1, 300]
    got = to_f64(run_prefix(wl, 256))
    assert np.isnan(got[3]).all()
    check(wl, got, exp, seqs=[0, 1, 2, 4, 5], label="prefix broken declaration")


def test_bad_block_id_in_the_prefix():
    # the longest sequence (1) is the row the prefix is read from; an id
    # outside the pool at page 100 makes every sequence that sees page 100
    # NaN (1 itself, and the others through the id mismatch), not 5 (L = 100)
    sp = spec("p_badid", 6, 32, 8, 128, "bf16", "bf16",
              ("fixed", [3000, 5000, 900, 4000, 4096, 100]), 4096, 21)
    wl = W.make_workload(sp)
    exp = ref(wl)
    t = to_device(wl)
    t["block_table"][1, 100] = wl.num_blocks + 3
    got = to_f64(run_prefix(wl, 256, t=t))
    for b in (0, 1, 3, 4):
        assert np.isnan(got[b]).all(), b
    check(wl, got, exp, seqs=[2, 5], label="prefix bad id")


def test_empty_and_out_of_contract_sequences():
    sp = spec("p_edge", 6, 8, 2, 128, "f16", "f16", ("fixed", [0, 5, 0, 700, 300, 2000]), 512, 22,
              mbs=130)
    wl = W.make_workload(sp)
    t = to_device(wl)
    t["context_lens"][4] = 130 * 16 + 1        # beyond the table
    t["context_lens"][2] = -3                  # negative
    B, Hq = wl.q.shape[:2]
    lse = torch.full((B, Hq), float("nan"), device="cuda")
    out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                     float(wl.scale), partition_size=BAL, lse_out=lse, prefix_blocks=32)
    torch.cuda.synchronize()
    got = to_f64(out)
    l = lse.cpu().numpy()
    assert np.array_equal(got[0], np.zeros_like(got[0])) and np.all(np.isneginf(l[0]))
    assert np.isnan(got[2]).all() and np.isnan(got[4]).all()
    check(wl, got, ref(wl), seqs=[1, 3, 5], label="prefix edge")


def test_deterministic_and_agrees_with_the_balanced_split_on_one_workspace():
    # The prefix call's counter region is the balanced split's, so the two
    # share one workspace in any order without a reset.
    sp = W.small_variant(W.SPECS[5], 8, ("loguniform", 100, 40000))
    wl = W.make_workload(sp, seed=23)
    t = to_device(wl)
    need = pkd.prefix_workspace_bytes(t["q"], t["k_cache"], t["block_table"])
    assert need >= pkd.workspace_bytes(t["q"], t["k_cache"], t["block_table"], BAL) > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    pkd.reset_workspace(ws)
    P = sp.shared_prefix_tokens // 16
    a = run_prefix(wl, P, t=t, workspace=ws).cpu()
    c = run(wl, t, partition_size=BAL, workspace=ws).cpu()
    b = run_prefix(wl, P, t=t, workspace=ws).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert np.abs(to_f64(a) - to_f64(c)).max() <= 2.5e-2
    check(wl, to_f64(a), ref(wl), label="prefix shared workspace")


def test_stale_counter_gives_nan_rows_until_reset():
    sp = spec("p_stale", 3, 8, 2, 128, "f16", "f16", ("fixed", [3000, 700, 2000]), 1024, 24)
    wl = W.make_workload(sp)
    t = to_device(wl)
    need = pkd.prefix_workspace_bytes(t["q"], t["k_cache"], t["block_table"])
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ws.view(torch.int32)[2] = 1000   # pair (1, 0)
    exp = ref(wl)
    G = 4
    for rep in range(2):
        out = to_f64(run_prefix(wl, 64, t=t, workspace=ws))
        assert np.isnan(out[1, :G]).all(), rep
        rest = np.concatenate([out[0].ravel(), out[1, G:].ravel(), out[2].ravel()])
        assert np.isfinite(rest).all()
        assert np.abs(out[0] - exp[0]).max() <= 1e-2 and np.abs(out[2] - exp[2]).max() <= 1e-2
    pkd.reset_workspace(ws)
    check(wl, to_f64(run_prefix(wl, 64, t=t, workspace=ws)), exp, label="prefix stale after reset")


def test_short_prefix_against_the_balanced_split_and_still_checked():
    # 8 shared pages of sequences 2000-4000 tokens long: little is saved,
    # the result is the plain balanced split's up to rounding, and the
    # declaration is still checked (a broken row: NaN for that sequence)
    sp = spec("p_small", 6, 32, 8, 128, "bf16", "bf16", ("uniform", 2000, 4000), 256, 25)
    wl = W.make_workload(sp)
    t = to_device(wl)
    a = to_f64(run_prefix(wl, 8, t=t))
    b = to_f64(run(wl, t, partition_size=BAL))
    assert np.abs(a - b).max() <= 2.5e-2
    exp = ref(wl)
    check(wl, a, exp, label="short prefix")
    # row 4 (not the longest, 2, whose ids are read) breaks it
    assert int(np.argmax(wl.context_lens)) == 2
    wl.block_table[4, 3] = wl.block_table[0, 40]
    got = to_f64(run_prefix(wl, 8))
    assert np.isnan(got[4]).all()
    check(wl, got, exp, seqs=[0, 1, 2, 3, 5], label="short prefix, declaration broken")


def random_prefix_config(seed):
    """A seeded shared-prefix configuration: any dtype pair and head_dim,
    1-8 KV heads, groups of 1-16, batches of 1-40, a shared prefix of 0-40
    blocks, sequences shorter than it (ending inside it or on its last page),
    empty, a whole table, and a declared prefix at, below or above the
    shared one (but never declaring more than the rows share)."""
    rng = np.random.default_rng(9100 + seed)
    DT = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3")]
    io, kv = DT[int(rng.integers(len(DT)))]
    D = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 17))
    B = int(rng.integers(1, 41))
    shared = int(rng.integers(0, 41))
    mbs = shared + int(rng.integers(1, 60))
    top = mbs * 16
    lens = []
    for kind in rng.integers(0, 6, size=B):
        lens.append([0, 16 * shared + int(rng.integers(1, 17)), top, int(rng.integers(1, top + 1)),
                     int(rng.integers(1, 16 * shared + 2)), 16 * int(rng.integers(1, mbs + 1))][int(kind)])
    declared = int(rng.integers(0, shared + 1)) if shared else 0
    sp = W.Spec(f"prand{seed}_{io}_{kv}_d{D}_h{G * hkv}kv{hkv}_b{B}_shared{shared}_P{declared}", B, G * hkv,
                hkv, D, io, kv, ("fixed", lens), mbs, ("ratio", 1.3), BAL, 16 * shared, 9100 + seed)
    return sp, declared


@pytest.mark.parametrize("seed", range(40))
def test_random_shared_prefix_configuration(seed):
    sp, P = random_prefix_config(seed)
    print(f"case {sp.name} lens={sp.lens[1]}", flush=True)
    wl = W.make_workload(sp)
    out, lse = run_prefix(wl, P, lse=True)
    exp_out, exp_lse = ref(wl, lse=True)
    got = to_f64(out)
    live = [b for b in range(sp.batch) if wl.context_lens[b] > 0]
    for b in range(sp.batch):
        if wl.context_lens[b] == 0:
            assert np.array_equal(got[b], np.zeros_like(got[b])), sp.name
    if live:
        check(wl, got, exp_out, seqs=live, label=sp.name)
        l = lse.cpu().double().numpy()
        assert np.array_equal(np.isneginf(l), np.isneginf(exp_lse)), sp.name
        fin = np.isfinite(exp_lse)
        assert np.abs(l[fin] - exp_lse[fin]).max() <= 5e-3, sp.name


def test_largest_batch_under_a_shared_prefix():
    # 4096 sequences of 1-200 tokens behind a 64-token prefix, 2 query heads
    # per KV head: 8 sequences per tile, 512 tiles, 128 passes per KV head;
    # the lengths scan covers the whole batch in LDS beside the prefix state
    sp = spec("p_b4096", 4096, 4, 2, 128, "bf16", "bf16", ("uniform", 1, 200), 64, 26)
    print(f"case {sp.name}", flush=True)
    wl = W.make_workload(sp)
    out = to_f64(run_prefix(wl, 4))
    exp = ref(wl)
    check(wl, out, exp, label="prefix largest batch")
