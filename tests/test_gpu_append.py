"""The paged KV append (pa_kv_append) against the oracle, bit for bit, on an
MI355X: every cache byte after the call must equal oracle/kv_append.py's
result on the same inputs (the bar for byte work), including the fp8 codes of
values planted at rounding ties, range edges, infinities and NaN. Then a
decode step (append the new token, attend over one more token) matches the
oracle doing the same two steps."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W
from paged_kv_decode_05_amd.workloads import _to_storage, storage_tensor
from tests.gpu_util import to_device, to_f64
from tests.test_gpu_parity import check, ref

pytestmark = pytest.mark.gpu


def special_values():
    """Values at every E4M3 rounding tie, the range edges, beyond the range,
    infinities, NaN, signed zeros and half the least subnormal."""
    pos = oracle.E4M3_TABLE[:127]
    mids = (pos[1:] + pos[:-1]) / 2
    return np.concatenate([mids, -mids, [0.0, -0.0, 448.0, -448.0, 449.0, 464.0, 480.0, 1e9,
                                         -1e9, np.inf, -np.inf, np.nan, 2.0 ** -10, -2.0 ** -10]])


def new_rows(rng, B, H, D, src, scales=None):
    """New K and V rows [B, H, D] in src storage; with scales (fp8 caches) the
    first elements of every row are planted with special_values() * scale."""
    x = rng.standard_normal((2, B, H, D)).astype(np.float32) * 2
    if scales is not None:
        vals = special_values()
        for which in range(2):
            for b in range(B):
                for h in range(H):
                    pick = rng.choice(len(vals), size=D // 2, replace=False)
                    x[which, b, h, : D // 2] = vals[pick] * float(scales[which][h])
    with np.errstate(over="ignore"):     # planted huge values overflow 16-bit storage to inf
        return _to_storage(x[0], src), _to_storage(x[1], src)


def give_new_blocks(wl, positions):
    """Point block_table[b][p // 16] at a free block of its own where the
    generator left it on the shared spare block, so no two sequences write
    the same (block, slot)."""
    used = set(np.unique(wl.block_table[wl.block_table >= 0]).tolist())
    spare = [b for b in range(wl.num_blocks) if b not in used]
    counts = np.bincount(wl.block_table.reshape(-1), minlength=wl.num_blocks)
    for b, p in enumerate(positions):
        if p < 0 or p >= 16 * wl.block_table.shape[1]:
            continue
        blk = wl.block_table[b, p // 16]
        if counts[blk] > 1:
            wl.block_table[b, p // 16] = spare.pop()


CASES = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
         ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3"), ("f32", "fp8_e4m3")]


@pytest.mark.parametrize("src,kv", CASES)
@pytest.mark.parametrize("D", [64, 128])
def test_append_is_bit_exact(src, kv, D):
    io = src if kv != "fp8_e4m3" else ("f16" if src == "f32" else src)
    spec = W.Spec(f"app_{src}_{kv}_{D}", 7, 8, 4, D, io, kv,
                  ("fixed", [0, 1, 15, 16, 31, 700, 2047]), 130, ("ratio", 1.3), 0, 0, D + 3)
    wl = W.make_workload(spec)
    rng = np.random.default_rng(D)
    ks = wl.k_scale if kv == "fp8_e4m3" else None
    vs = wl.v_scale if kv == "fp8_e4m3" else None
    k_new, v_new = new_rows(rng, 7, 4, D, src, (ks, vs) if ks is not None else None)
    pos = wl.context_lens.astype(np.int32).copy()
    pos[3] = -1                       # padding row: nothing written
    pos[5] = 130 * 16 + 3             # past the table: nothing written
    give_new_blocks(wl, pos)
    t = to_device(wl)
    print(f"case {spec.name}", flush=True)
    pkd.kv_append(storage_tensor(k_new, src).cuda(), storage_tensor(v_new, src).cuda(),
                  torch.from_numpy(pos).cuda(), t["block_table"], t["k_cache"], t["v_cache"],
                  k_scale=t["k_scale"], v_scale=t["v_scale"])
    torch.cuda.synchronize()
    want_k, want_v = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new, wl.block_table,
                                          pos, src, kv, ks, vs)
    got_k = t["k_cache"].cpu().contiguous().view(torch.uint8).numpy()
    got_v = t["v_cache"].cpu().contiguous().view(torch.uint8).numpy()
    bk = np.ascontiguousarray(want_k).view(np.uint8).reshape(got_k.shape)
    bv = np.ascontiguousarray(want_v).view(np.uint8).reshape(got_v.shape)
    nk, nv = int((got_k != bk).sum()), int((got_v != bv).sum())
    print(f"  differing bytes K {nk} V {nv}", flush=True)
    assert nk == 0 and nv == 0


def test_out_of_range_block_writes_nothing():
    spec = W.Spec("app_badblk", 3, 4, 2, 128, "f16", "f16", ("fixed", [5, 40, 70]), 8,
                  ("ratio", 1.5), 0, 0, 9)
    wl = W.make_workload(spec)
    t = to_device(wl)
    before_k, before_v = t["k_cache"].clone(), t["v_cache"].clone()
    k_new, v_new = new_rows(np.random.default_rng(1), 3, 2, 128, "f16")
    bt = t["block_table"].clone()
    bt[:, :] = wl.num_blocks + 3
    pkd.kv_append(storage_tensor(k_new, "f16").cuda(), storage_tensor(v_new, "f16").cuda(),
                  torch.from_numpy(wl.context_lens.astype(np.int32)).cuda(), bt, t["k_cache"],
                  t["v_cache"])
    torch.cuda.synchronize()
    assert torch.equal(t["k_cache"].view(torch.int16), before_k.view(torch.int16))
    assert torch.equal(t["v_cache"].view(torch.int16), before_v.view(torch.int16))


@pytest.mark.parametrize("io,kv,ps", [("f16", "f16", 512), ("bf16", "fp8_e4m3", pkd.SPLIT_BALANCED),
                                      ("f16", "fp8_e4m3", 0)])
def test_decode_step_append_then_attend(io, kv, ps):
    # A decode step: append the new token at position L, then attend over
    # L + 1 tokens; compare with the oracle doing the same two steps.
    base = W.SPECS[4] if kv == "fp8_e4m3" else W.SPECS[3]
    spec = W.Spec(f"step_{io}_{kv}_{ps}", 5, base.num_q_heads, base.num_kv_heads, 128, io, kv,
                  ("uniform", 30, 1500), 100, ("ratio", 1.3), ps, 0, 17)
    wl = W.make_workload(spec)
    L = wl.context_lens.astype(np.int32)
    give_new_blocks(wl, L)
    t = to_device(wl)
    ks = wl.k_scale if kv == "fp8_e4m3" else None
    vs = wl.v_scale if kv == "fp8_e4m3" else None
    k_new, v_new = new_rows(np.random.default_rng(4), spec.batch, spec.num_kv_heads, 128, io)
    print(f"case {spec.name}", flush=True)
    pkd.kv_append(storage_tensor(k_new, io).cuda(), storage_tensor(v_new, io).cuda(),
                  torch.from_numpy(L).cuda(), t["block_table"], t["k_cache"], t["v_cache"],
                  k_scale=t["k_scale"], v_scale=t["v_scale"])
    lens = torch.from_numpy(L + 1).cuda()
    out = pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], lens,
                     float(wl.scale), k_scale=t["k_scale"], v_scale=t["v_scale"], partition_size=ps)
    torch.cuda.synchronize()
    kc, vc = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new, wl.block_table, L, io, kv,
                                  ks, vs)
    wl.k_cache, wl.v_cache, wl.context_lens = kc, vc, L + 1
    check(wl, to_f64(out), ref(wl), label=f"append+decode {io}/{kv} ps{ps}")
