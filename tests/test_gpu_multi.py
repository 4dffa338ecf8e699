"""Multi-token query attention (pa_decode_multi) against the float64 oracle
(oracle/multi_query.py) on an MI355X: q_len new tokens per sequence, causal
among themselves, over the paged cache. Same bar as decode (tests/
test_gpu_parity.py): max-abs 1e-2 / mean-abs 1e-3, fp8 caches 3e-2 / 3e-3.
Cases span every dtype pair and head_dim, 1 to 16 new tokens, group sizes
1 to 16 (16 to 256 query rows per KV head: one to eight row chunks), split
partitions that some rows see nothing of, sequences shorter than q_len,
empty and out-of-contract metadata, and a verify step that appends the new
tokens first."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from paged_kv_decode_05_amd.workloads import storage_tensor
from tests.gpu_util import to_device, to_f64
from tests.test_gpu_append import give_new_blocks, new_rows
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


def run_multi(wl, q, t=None, ps=None, lse=False, workspace=None, lens=None):
    t = t or to_device(wl)
    ps = wl.spec.partition_size if ps is None else ps
    qt = storage_tensor(q, wl.spec.io_dtype).cuda()
    lse_out = torch.full(q.shape[:3], float("nan"), device="cuda") if lse else None
    cl = t["context_lens"] if lens is None else lens
    out = pkd.decode(qt, t["k_cache"], t["v_cache"], t["block_table"], cl, float(wl.scale),
                     k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=ps,
                     workspace=workspace, lse_out=lse_out)
    torch.cuda.synchronize()
    return (out, lse_out) if lse else out


def ref_multi(wl, q, lse=False, seqs=None):
    return oracle.multi_query_ref(q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens,
                                  wl.scale, wl.spec.io_dtype, wl.spec.kv_dtype, wl.k_scale,
                                  wl.v_scale, return_lse=lse, seqs=seqs)


def spec_of(name, io, kv, D, lens, hq=8, hkv=2, mbs=None, ps=0, seed=3):
    top = max(lens)
    mbs = mbs or max(1, -(-top // 16))
    return W.Spec(name, len(lens), hq, hkv, D, io, kv, ("fixed", list(lens)), mbs,
                  ("ratio", 1.3), ps, 0, seed)


DTYPES = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8_e4m3"),
          ("bf16", "fp8_e4m3")]


@pytest.mark.parametrize("io,kv", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("ps", [0, 64])
def test_dtype_headdim_matrix(io, kv, D, ps):
    spec = spec_of(f"mq_{io}_{kv}_{D}_{ps}", io, kv, D, [1, 3, 17, 100, 700], ps=ps)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 4)
    out, lse = run_multi(wl, q, lse=True)
    exp, rlse = ref_multi(wl, q, lse=True)
    check(wl, to_f64(out), exp, label=spec.name)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.abs(l[fin] - rlse[fin]).max() <= 2e-3


@pytest.mark.parametrize("T", [1, 2, 3, 7, 16])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (28, 4), (32, 2)])
def test_query_lengths_and_groups(T, hq, hkv):
    # G * T from 1 to 256 rows: one to eight row chunks of up to 32 rows
    spec = spec_of(f"mq_T{T}_g{hq // hkv}", "f16", "f16", 128, [5, 16, 300, 1111], hq=hq,
                   hkv=hkv, ps=512, seed=T)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, T)
    check(wl, to_f64(run_multi(wl, q)), ref_multi(wl, q), label=spec.name)


@pytest.mark.parametrize("ps", [16, 512])
def test_partitions_some_rows_cannot_see(ps):
    # L = 520 with 16 new tokens: new token 0 sees 0 .. 504, so with
    # 512-token partitions the second partition is empty for it; with 16-token
    # partitions the last page's partition is empty for the first tokens.
    spec = spec_of(f"mq_part_{ps}", "bf16", "bf16", 128, [520, 513, 528, 16], ps=ps, seed=8)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 16)
    out, lse = run_multi(wl, q, lse=True)
    exp, rlse = ref_multi(wl, q, lse=True)
    check(wl, to_f64(out), exp, label=spec.name)
    fin = np.isfinite(rlse)
    assert np.abs(lse.cpu().numpy()[fin] - rlse[fin]).max() <= 2e-3


@pytest.mark.parametrize("T", [2, 4, 8])
def test_two_level_merge(T):
    # 16-token partitions, up to 66 per sequence: groups of 16 partitions
    # merge first, then the groups. G = 4: T = 2 and 4 run on the decode
    # kernels, T = 8 (32 rows) on the multi-token kernel. At 1025 and 257
    # tokens the last group is one partition holding only the last position,
    # which no new token but the last may see; at 7 tokens the first new
    # tokens see nothing at all.
    spec = spec_of(f"mq_tree_T{T}", "bf16", "bf16", 128, [1025, 1056, 272, 257, 7], ps=16,
                   seed=20 + T)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, T)
    out, lse = run_multi(wl, q, lse=True)
    exp, rlse = ref_multi(wl, q, lse=True)
    check(wl, to_f64(out), exp, label=spec.name)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.abs(l[fin] - rlse[fin]).max() <= 2e-3


def test_one_new_token_equals_decode():
    spec = spec_of("mq_t1", "f16", "f16", 128, [1, 40, 513, 2000], ps=512, seed=4)
    wl = W.make_workload(spec)
    t = to_device(wl)
    q1 = W.multi_query(wl, 1)
    for ps in (0, 512):
        got = run_multi(wl, q1, t=t, ps=ps)
        dec = pkd.decode(storage_tensor(np.ascontiguousarray(q1[:, 0]), "f16").cuda(),
                         t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                         float(wl.scale), partition_size=ps)
        torch.cuda.synchronize()
        # same pages, masks and merges as the decode kernel: bit for bit
        assert torch.equal(got[:, 0].cpu().view(torch.int16), dec.cpu().view(torch.int16)), ps


def test_full_size_qwen7b_shape_verify_step():
    # The Qwen2.5-7B-shaped workload (32 sequences, 28/4 heads, 512-4096
    # tokens, 512-token partitions) with 8 new tokens per sequence; the oracle
    # checks a sample of sequences.
    spec = W.SPECS[3]
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 8)
    print(f"case full {spec.name} T=8", flush=True)
    out = to_f64(run_multi(wl, q))
    assert np.isfinite(out).all()
    seqs = [0, 7, 19, 31]
    check(wl, out, ref_multi(wl, q, seqs=seqs), seqs=seqs, label="full-T8")


def test_fp8_long_context_shape_sampled():
    spec = W.SPECS[4]
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 4)
    print(f"case full {spec.name} T=4", flush=True)
    out = to_f64(run_multi(wl, q))
    assert np.isfinite(out).all()
    seqs = [3, 64, 127]
    check(wl, out, ref_multi(wl, q, seqs=seqs), seqs=seqs, label="fp8-T4")


def test_empty_and_out_of_contract_metadata():
    spec = spec_of("mq_meta", "f16", "f16", 128, [0, 100, 200, 300, 50], ps=64, seed=5)
    wl = W.make_workload(spec)
    t = to_device(wl)
    t["context_lens"][1] = wl.block_table.shape[1] * 16 + 1       # beyond the table
    t["block_table"][2, 3] = wl.num_blocks + 1000                  # beyond the pool
    q = W.multi_query(wl, 5)
    out, lse = run_multi(wl, q, t=t, lse=True)
    got = to_f64(out)
    l = lse.cpu().numpy()
    assert (got[0] == 0).all() and np.isneginf(l[0]).all()
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    check(wl, got, ref_multi(wl, q, seqs=[3, 4]), seqs=[3, 4], label="meta-ok-seqs")


def test_workspace_shared_across_query_lengths():
    spec = spec_of("mq_ws", "bf16", "bf16", 128, [100, 900, 2000, 333], ps=256, seed=6)
    wl = W.make_workload(spec)
    t = to_device(wl)
    qs = {T: W.multi_query(wl, T) for T in (16, 3, 1)}
    big = storage_tensor(qs[16], "bf16").cuda()
    need = pkd.workspace_bytes(big, t["k_cache"], t["block_table"], 256)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    pkd.reset_workspace(ws)
    for rnd in range(2):
        for T in (16, 3, 1):
            check(wl, to_f64(run_multi(wl, qs[T], t=t, workspace=ws)), ref_multi(wl, qs[T]),
                  label=f"ws T{T} round{rnd}")


def test_run_to_run_bit_determinism():
    spec = spec_of("mq_det", "f16", "fp8_e4m3", 128, [3000, 17, 999], ps=512, seed=7)
    wl = W.make_workload(spec)
    t = to_device(wl)
    q = W.multi_query(wl, 6)
    a = run_multi(wl, q, t=t).cpu()
    b = run_multi(wl, q, t=t).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("io,kv,ps", [("f16", "f16", 512), ("bf16", "fp8_e4m3", 0)])
def test_verify_step_append_then_attend(io, kv, ps):
    # Speculative verify / chunked-prefill tail: append T new tokens' K/V at
    # positions L .. L+T-1 (one pa_kv_append per token), then attend with
    # lengths L+T; the oracle does the same steps.
    T = 5
    spec = W.Spec(f"verify_{io}_{kv}_{ps}", 5, 28, 4, 128, io, kv, ("uniform", 30, 1500), 100,
                  ("ratio", 1.4), ps, 0, 23)
    wl = W.make_workload(spec)
    t = to_device(wl)
    L0 = wl.context_lens.astype(np.int32)
    ks = wl.k_scale if kv == "fp8_e4m3" else None
    vs = wl.v_scale if kv == "fp8_e4m3" else None
    rng = np.random.default_rng(9)
    print(f"case {spec.name}", flush=True)
    for i in range(T):
        pos = L0 + i
        give_new_blocks(wl, pos)
        t["block_table"].copy_(torch.from_numpy(wl.block_table))
        k_new, v_new = new_rows(rng, spec.batch, spec.num_kv_heads, 128, io)
        pkd.kv_append(storage_tensor(k_new, io).cuda(), storage_tensor(v_new, io).cuda(),
                      torch.from_numpy(pos).cuda(), t["block_table"], t["k_cache"],
                      t["v_cache"], k_scale=t["k_scale"], v_scale=t["v_scale"])
        wl.k_cache, wl.v_cache = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new,
                                                      wl.block_table, pos, io, kv, ks, vs)
    wl.context_lens = L0 + T
    q = W.multi_query(wl, T)
    out = run_multi(wl, q, t=t, lens=torch.from_numpy(wl.context_lens).cuda())
    check(wl, to_f64(out), ref_multi(wl, q), label=spec.name)


def test_largest_batch_and_rows_sampled():
    # 2048 sequences of up to 40 tokens, 16 query heads on one KV head and 16
    # new tokens: 256 rows (eight chunks) per pair, 16384 workgroups in one
    # pass; the oracle checks a sample of sequences (all the short ones too)
    spec = W.Spec("mq_large", 2048, 16, 1, 64, "bf16", "bf16", ("uniform", 0, 40), 3,
                  ("ratio", 1.2), 0, 0, 41)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 16)
    print(f"case {spec.name}", flush=True)
    out = to_f64(run_multi(wl, q))
    seqs = sorted(set([0, 1, 777, 2047] + [int(b) for b in np.nonzero(wl.context_lens < 16)[0][:8]]))
    check(wl, out, ref_multi(wl, q, seqs=seqs), seqs=seqs, label="large")


@pytest.mark.parametrize("io,kv", DTYPES)
@pytest.mark.parametrize("hq,hkv,T", [(8, 2, 4), (8, 4, 8), (28, 4, 2), (16, 1, 1), (8, 8, 16)])
def test_balanced_split_when_rows_fit_one_tile(io, kv, hq, hkv, T):
    # G * T <= 16: the decode kernels run the call; the balanced split cuts
    # the pairs' pages into equal shares, including the pages that hold
    # the new tokens (causal masks) and sequences shorter than T
    spec = spec_of(f"mq_bal_{io}_{kv}_{hq}_{hkv}_{T}", io, kv, 128, [1, 3, 17, 100, 700, 2047],
                   hq=hq, hkv=hkv, ps=-1, seed=T + hq)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, T)
    out, lse = run_multi(wl, q, lse=True)
    exp, rlse = ref_multi(wl, q, lse=True)
    check(wl, to_f64(out), exp, label=spec.name)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.abs(l[fin] - rlse[fin]).max() <= 2e-3


@pytest.mark.parametrize("ps", [-1, 0, 512])
def test_tile_rows_long_context_shape_sampled(ps):
    # the long-context workload (Llama-3-8B shape, G = 4) with four new
    # tokens: 16 rows, the decode kernels in all three split modes
    spec = W.SPECS[5]
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 4)
    print(f"case full {spec.name} T=4 ps{ps}", flush=True)
    out = to_f64(run_multi(wl, q, ps=ps))
    assert np.isfinite(out).all()
    seqs = [0, 3, 7]
    check(wl, out, ref_multi(wl, q, seqs=seqs), seqs=seqs, label=f"long-T4-ps{ps}")


def test_tile_rows_split_modes_agree_and_t1_is_decode_in_every_mode():
    spec = spec_of("mq_modes", "f16", "f16", 128, [5, 600, 1500, 33], ps=512, seed=13)
    wl = W.make_workload(spec)
    t = to_device(wl)
    q = W.multi_query(wl, 4)
    outs = [to_f64(run_multi(wl, q, t=t, ps=ps)) for ps in (0, 512, -1)]
    assert np.abs(outs[0] - outs[1]).max() <= 2e-3 and np.abs(outs[0] - outs[2]).max() <= 2e-3
    q1 = W.multi_query(wl, 1)
    for ps in (0, 512, -1):
        got = run_multi(wl, q1, t=t, ps=ps)
        dec = pkd.decode(storage_tensor(np.ascontiguousarray(q1[:, 0]), "f16").cuda(),
                         t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                         float(wl.scale), partition_size=ps)
        torch.cuda.synchronize()
        assert torch.equal(got[:, 0].cpu().view(torch.int16), dec.cpu().view(torch.int16)), ps


# ---- the balanced split for rows wider than one tile (G * T > 16) ----------
# Cases by row chunks (two 16-row tiles each): one chunk (all four waves on
# it), two chunks (two waves each), three and four chunks (a wave each), and
# more than four (two passes over each piece).
WIDE = [(4, 1, 8, 1), (8, 1, 8, 2), (28, 4, 8, 2), (8, 1, 12, 3), (28, 4, 16, 4), (16, 1, 16, 8)]


@pytest.mark.parametrize("hq,hkv,T,chunks", WIDE)
def test_balanced_wide_rows_every_chunk_count(hq, hkv, T, chunks):
    G = hq // hkv
    assert -(-(G * T) // 32) == chunks and G * T > 16
    spec = spec_of(f"mq_balw_{hq}_{hkv}_{T}", "f16", "f16", 128, [1, 3, 17, 100, 700, 2047, 5000],
                   hq=hq, hkv=hkv, ps=-1, seed=T + 3 * hq)
    print(f"case {spec.name} chunks={chunks}", flush=True)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, T)
    out, lse = run_multi(wl, q, lse=True)
    exp, rlse = ref_multi(wl, q, lse=True)
    check(wl, to_f64(out), exp, label=spec.name)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(l), np.isneginf(rlse))
    fin = np.isfinite(rlse)
    assert np.abs(l[fin] - rlse[fin]).max() <= 2e-3


@pytest.mark.parametrize("io,kv", DTYPES)
@pytest.mark.parametrize("D", [64, 128])
def test_balanced_wide_rows_dtypes_and_head_dims(io, kv, D):
    spec = spec_of(f"mq_balw_{io}_{kv}_{D}", io, kv, D, [2, 40, 333, 1200, 2900], hq=8, hkv=2,
                   ps=-1, seed=11)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 7)        # 28 rows: two tiles
    check(wl, to_f64(run_multi(wl, q)), ref_multi(wl, q), label=spec.name)
    q = W.multi_query(wl, 16)       # 64 rows: two chunks
    check(wl, to_f64(run_multi(wl, q)), ref_multi(wl, q), label=spec.name + "-T16")


def test_balanced_wide_rows_one_pair_over_many_shares_and_many_short_pairs():
    # one sequence far longer than the rest (its pairs are cut into many
    # pieces, each share merging partials) and a batch of short sequences
    # (a share walks many whole pairs)
    lens = [30000, 7] + [int(x) for x in np.random.default_rng(5).integers(1, 120, 150)]
    spec = spec_of("mq_balw_mix", "bf16", "bf16", 128, lens, hq=16, hkv=2, ps=-1, seed=21)
    print(f"case {spec.name}", flush=True)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, 5)        # 40 rows: two chunks
    out = to_f64(run_multi(wl, q))
    seqs = [0, 1, 2, 50, 151]
    check(wl, out, ref_multi(wl, q, seqs=seqs), seqs=seqs, label=spec.name)
    assert np.isfinite(out).all()


def test_balanced_wide_rows_metadata_and_determinism():
    spec = spec_of("mq_balw_meta", "f16", "fp8_e4m3", 128, [0, 100, 200, 3000, 50], ps=-1, seed=9)
    wl = W.make_workload(spec)
    t = to_device(wl)
    t["context_lens"][1] = wl.block_table.shape[1] * 16 + 1       # beyond the table
    t["block_table"][2, 3] = wl.num_blocks + 1000                  # beyond the pool
    q = W.multi_query(wl, 6)        # 24 rows
    out, lse = run_multi(wl, q, t=t, lse=True)
    got = to_f64(out)
    l = lse.cpu().numpy()
    assert (got[0] == 0).all() and np.isneginf(l[0]).all()
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    check(wl, got, ref_multi(wl, q, seqs=[3, 4]), seqs=[3, 4], label="balw-meta-ok-seqs")
    for i in range(5):
        again = run_multi(wl, q, t=t)
        assert torch.equal(out.cpu().view(torch.int16), again.cpu().view(torch.int16)), i


def test_balanced_wide_rows_stale_counter_gives_nan_rows_until_reset():
    spec = spec_of("mq_balw_stale", "f16", "f16", 128, [6000, 700], hq=8, hkv=2, ps=-1, seed=4)
    wl = W.make_workload(spec)
    t = to_device(wl)
    q = W.multi_query(wl, 8)        # 32 rows
    qt = storage_tensor(q, "f16").cuda()
    ws = torch.zeros(pkd.workspace_bytes(qt, t["k_cache"], t["block_table"], -1),
                     dtype=torch.uint8, device="cuda")
    exp = ref_multi(wl, q)
    ws.view(torch.int32)[0] = 1000          # counter of pair (0, 0): far beyond its pieces
    G = spec.num_q_heads // spec.num_kv_heads
    for rep in range(2):
        out = to_f64(run_multi(wl, q, t=t, workspace=ws))
        assert np.isnan(out[0, :, :G]).all(), rep                      # pair (0, 0), every new token
        assert np.isfinite(out[0, :, G:]).all() and np.isfinite(out[1]).all()
        assert np.abs(out[1] - exp[1]).max() <= 1e-2
    pkd.reset_workspace(ws)
    check(wl, to_f64(run_multi(wl, q, t=t, workspace=ws)), exp, label="balw stale after reset")


def test_balanced_wide_rows_full_size_qwen7b_shape_sampled():
    # the Qwen2.5-7B-shaped workload with 8 and 16 new tokens per sequence in
    # the balanced split (the mode bench.py times for it)
    spec = W.SPECS[3]
    wl = W.make_workload(spec)
    for T in (8, 16):
        q = W.multi_query(wl, T)
        print(f"case full {spec.name} T={T} balanced", flush=True)
        out = to_f64(run_multi(wl, q, ps=-1))
        assert np.isfinite(out).all()
        seqs = [0, 7, 19, 31]
        check(wl, out, ref_multi(wl, q, seqs=seqs), seqs=seqs, label=f"full-T{T}-bal")
