"""Pins for the float64 oracle: brute force, a library routine, closed forms,
invariants and planted mistakes. All CPU-only.

The pages print no worked example for this path, so the oracle is pinned by
(1) a pure-Python brute force on tiny inputs, (2) torch's scaled-dot-product
attention (float64, grouped-query) on contiguous gathers built by explicit
index arithmetic, (3) closed forms of special cases, and (4) invariants of the
method: permuting physical blocks together with the block table, split-K with
a log-sum-exp merge, a one-token context, identical V rows, a zero query.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_05_amd import workloads as W
from tests.brute import brute_decode


def tiny_spec(io, kv, B=3, hq=4, hkv=2, D=16, lens=("fixed", [5, 16, 37]),
              mbs=4, pool=("fixed", 14), ps=0, prefix=0, seed=11):
    return W.Spec(f"tiny_{io}_{kv}", B, hq, hkv, D, io, kv, lens, mbs, pool, ps, prefix, seed)


DTYPES = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("f16", "fp8_e4m3"),
          ("bf16", "fp8_e4m3")]


def run_oracle(wl, **kw):
    return oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                   wl.context_lens, wl.scale, wl.spec.io_dtype,
                                   wl.spec.kv_dtype, wl.k_scale, wl.v_scale, **kw)


# ---------------------------------------------------------------- formats

def test_e4m3_table_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_TABLE
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x38] == 1.0


def test_half_and_bfloat_decoders_match_torch():
    rng = np.random.default_rng(0)
    words = rng.integers(0, 1 << 16, size=20000, dtype=np.uint32).astype(np.uint16)
    words[:6] = [0x0000, 0x8000, 0x0001, 0x7C00, 0x7E00, 0x3C00]
    t = torch.from_numpy(words.view(np.int16))
    for name, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        ref = t.view(tdt).to(torch.float64).numpy()
        ours = oracle.decode(words, name)
        same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
        assert same.all(), name


def test_generator_fp8_quantizer_round_trip():
    # every finite code decodes to a value that quantizes back to itself
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = oracle.E4M3_TABLE[finite].astype(np.float32)
    codes = W._to_e4m3(vals, np.float32(1.0))
    back = oracle.E4M3_TABLE[codes]
    assert np.array_equal(back, oracle.E4M3_TABLE[finite])
    # out-of-range values saturate instead of turning into NaN
    big = W._to_e4m3(np.array([500.0, -1e9, 449.0, 464.1], dtype=np.float32), np.float32(1.0))
    assert list(oracle.E4M3_TABLE[big]) == [448.0, -448.0, 448.0, 448.0]


# ------------------------------------------------------- brute force (P1)

@pytest.mark.parametrize("io,kv", DTYPES)
def test_oracle_matches_brute_force(io, kv):
    wl = W.make_workload(tiny_spec(io, kv))
    out, lse = run_oracle(wl, return_lse=True)
    bout, blse = brute_decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                              wl.context_lens, wl.scale, io, kv, wl.k_scale, wl.v_scale)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_oracle_matches_brute_force_gqa_shapes():
    for hq, hkv in ((6, 2), (3, 1), (4, 4)):
        wl = W.make_workload(tiny_spec("f16", "f16", hq=hq, hkv=hkv, seed=hq * 7 + hkv))
        out, lse = run_oracle(wl, return_lse=True)
        bout, blse = brute_decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                  wl.context_lens, wl.scale, "f16", "f16")
        np.testing.assert_allclose(out, bout, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, blse, rtol=0, atol=1e-12)


def test_oracle_matches_brute_force_on_tiny_workload_one():
    # The tiny fp32 workload at its real shape (B4, 8/2 heads, D64, lengths
    # 1, 17, 100, 256); the brute force covers the two shortest sequences.
    wl = W.make_workload(W.SPECS[1])
    out, lse = run_oracle(wl, return_lse=True)
    sub = slice(0, 2)
    bout, blse = brute_decode(wl.q[sub], wl.k_cache, wl.v_cache, wl.block_table[sub],
                              wl.context_lens[sub], wl.scale, "f32", "f32")
    np.testing.assert_allclose(out[sub], bout, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[sub], blse, rtol=0, atol=1e-12)


# ------------------------------------------------ library routine (P2)

def explicit_gather(wl, b, g, dtype_scale=True):
    """Contiguous K, V rows [L, D] of (b, g) by flat-index arithmetic."""
    s = wl.spec
    D, Hkv, x = s.head_dim, s.num_kv_heads, wl.x
    L = int(wl.context_lens[b])
    t = np.arange(L)
    blk = wl.block_table[b][t // 16].astype(np.int64)[:, None]
    d = np.arange(D)[None, :]
    kidx = ((((blk * Hkv + g) * (D // x) + d // x) * 16 + (t % 16)[:, None]) * x + d % x)
    vidx = (((blk * Hkv + g) * D + d) * 16 + (t % 16)[:, None])
    K = torch.from_numpy(wl.k_cache.reshape(-1)[kidx].copy())
    V = torch.from_numpy(wl.v_cache.reshape(-1)[vidx].copy())
    return K, V


def torch_decode(raw, dtype):
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == "f32":
        return t.to(torch.float64)
    if dtype == "f16":
        return t.view(torch.int16).view(torch.float16).to(torch.float64)
    if dtype == "bf16":
        return t.view(torch.int16).view(torch.bfloat16).to(torch.float64)
    return t.view(torch.float8_e4m3fn).to(torch.float64)


@pytest.mark.parametrize("io,kv", DTYPES)
def test_oracle_matches_torch_sdpa(io, kv):
    spec = tiny_spec(io, kv, B=3, hq=8, hkv=2, D=64, lens=("fixed", [1, 40, 130]),
                     mbs=9, pool=("fixed", 20), seed=5)
    wl = W.make_workload(spec)
    out, lse = run_oracle(wl, return_lse=True)
    qall = torch_decode(wl.q, io)
    for b in range(spec.batch):
        Ks, Vs = [], []
        for g in range(spec.num_kv_heads):
            K, V = explicit_gather(wl, b, g)
            K, V = torch_decode(K.numpy(), kv), torch_decode(V.numpy(), kv)
            if kv == "fp8_e4m3":
                K = K * float(wl.k_scale[g])
                V = V * float(wl.v_scale[g])
            Ks.append(K)
            Vs.append(V)
        K = torch.stack(Ks)[None]          # [1, Hkv, L, D]
        V = torch.stack(Vs)[None]
        qb = qall[b][None, :, None, :]     # [1, Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qb, K, V, scale=float(wl.scale), enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------- closed forms

def handmade(io="f32", D=64, L=2, hq=1, hkv=1, nb=4):
    spec = tiny_spec(io, io, B=1, hq=hq, hkv=hkv, D=D, lens=("fixed", [L]),
                     mbs=max(1, -(-L // 16)), pool=("fixed", nb), seed=3)
    return W.make_workload(spec, poison=False)


def test_closed_form_two_tokens():
    # Two keys with scores a, b: out = sigmoid(a-b) v0 + sigmoid(b-a) v1.
    wl = handmade(L=2)
    blk = int(wl.block_table[0, 0])
    out, lse = run_oracle(wl, return_lse=True)
    K, V = explicit_gather(wl, 0, 0)
    q = wl.q[0, 0].astype(np.float64)
    sc = float(wl.scale)
    K, V = K.numpy().astype(np.float64), V.numpy().astype(np.float64)
    a, b = sc * float(q @ K[0]), sc * float(q @ K[1])
    w0 = 1.0 / (1.0 + math.exp(b - a))
    expect = w0 * V[0] + (1.0 - w0) * V[1]
    np.testing.assert_allclose(out[0, 0], expect, rtol=0, atol=1e-12)
    assert abs(lse[0, 0] - (max(a, b) + math.log1p(math.exp(-abs(a - b))))) < 1e-12
    assert blk == wl.block_table[0, 0]


def test_one_token_context_returns_v():
    for io, kv in DTYPES:
        spec = tiny_spec(io, kv, lens=("fixed", [1, 1, 17]))
        wl = W.make_workload(spec)
        out = run_oracle(wl)
        for b in (0, 1):
            for h in range(4):
                g = h // 2
                _, V = explicit_gather(wl, b, g)
                v = torch_decode(V.numpy(), kv)[0].numpy()
                if kv == "fp8_e4m3":
                    v = v * float(wl.v_scale[g])
                assert np.array_equal(out[b, h], v)


def test_identical_v_rows_return_that_row():
    spec = tiny_spec("f16", "f16", lens=("fixed", [9, 33, 64]), mbs=4, pool=("fixed", 14))
    wl = W.make_workload(spec, poison=False)
    row = np.random.default_rng(1).standard_normal(16).astype(np.float16).view(np.uint16)
    wl.v_cache[:] = row[None, None, :, None]
    out = run_oracle(wl)
    np.testing.assert_allclose(out, np.broadcast_to(row.view(np.float16).astype(np.float64),
                                                    out.shape), rtol=1e-15, atol=0)


def test_zero_query_gives_mean_of_values():
    spec = tiny_spec("f32", "f32", lens=("fixed", [3, 20, 47]), mbs=4, pool=("fixed", 14))
    wl = W.make_workload(spec)
    wl.q[:] = 0
    out, lse = run_oracle(wl, return_lse=True)
    for b in range(3):
        L = int(wl.context_lens[b])
        for h in range(4):
            _, V = explicit_gather(wl, b, h // 2)
            np.testing.assert_allclose(out[b, h], V.numpy().astype(np.float64).mean(0),
                                       rtol=0, atol=1e-13)
            assert abs(lse[b, h] - math.log(L)) < 1e-13


def test_empty_context_convention():
    spec = tiny_spec("f16", "f16", lens=("fixed", [0, 5, 0]))
    wl = W.make_workload(spec)
    out, lse = run_oracle(wl, return_lse=True)
    assert np.array_equal(out[0], np.zeros_like(out[0])) and np.all(lse[0] == -np.inf)
    assert np.array_equal(out[2], np.zeros_like(out[2]))
    assert np.isfinite(out[1]).all()


# ---------------------------------------------------------- invariants

@pytest.mark.parametrize("io,kv", DTYPES)
def test_block_permutation_invariance(io, kv):
    spec = tiny_spec(io, kv, B=3, hq=8, hkv=2, D=64, lens=("fixed", [7, 48, 100]),
                     mbs=7, pool=("fixed", 20), seed=9)
    wl = W.make_workload(spec)
    out = run_oracle(wl)
    pi = np.random.default_rng(2).permutation(wl.num_blocks)
    k2 = np.empty_like(wl.k_cache)
    v2 = np.empty_like(wl.v_cache)
    k2[pi] = wl.k_cache
    v2[pi] = wl.v_cache
    t2 = pi[wl.block_table].astype(np.int32)
    out2 = oracle.paged_decode_ref(wl.q, k2, v2, t2, wl.context_lens, wl.scale, io, kv,
                                   wl.k_scale, wl.v_scale)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("ps", [16, 32, 48, 512])
def test_split_merge_equals_unsplit(ps):
    spec = tiny_spec("bf16", "bf16", B=3, hq=8, hkv=2, D=64, lens=("fixed", [16, 97, 300]),
                     mbs=19, pool=("fixed", 40), seed=ps)
    wl = W.make_workload(spec)
    out, lse = run_oracle(wl, return_lse=True)
    sout, slse = oracle.paged_decode_split_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                               wl.context_lens, wl.scale, "bf16", "bf16", ps)
    np.testing.assert_allclose(sout, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(slse, lse, rtol=0, atol=1e-12)


def test_lse_merge_ignores_empty_partials():
    o = np.array([[1.0, 2.0], [5.0, 7.0]])
    out, lse = oracle.lse_merge(o, np.array([0.3, -np.inf]))
    assert np.array_equal(out, o[0]) and lse == 0.3
    out, lse = oracle.lse_merge(o, np.array([-np.inf, -np.inf]))
    assert np.array_equal(out, [0.0, 0.0]) and lse == -np.inf


def test_poison_never_reaches_output_and_lands_where_claimed():
    spec = tiny_spec("f16", "f16", lens=("fixed", [5, 16, 37]))
    wl = W.make_workload(spec)
    # the generator put NaN in the spare block and in every unread tail slot
    assert np.isnan(oracle.decode(wl.k_cache[wl.spare_block], "f16")).all()
    assert np.isfinite(run_oracle(wl)).all()
    # a NaN planted in the last valid slot does reach the output
    b, L = 2, 37
    blk = int(wl.block_table[b, (L - 1) // 16])
    bad = W.make_workload(spec)
    bad.v_cache[blk, 0, :, (L - 1) % 16] = W.NAN_BITS["f16"]
    o = run_oracle(bad)
    assert np.isnan(o[b, :2]).all() and np.isfinite(o[b, 2:]).all()


def test_equal_queries_in_a_group_give_equal_outputs():
    spec = tiny_spec("f16", "f16", B=2, hq=8, hkv=2, D=64, lens=("fixed", [40, 70]),
                     mbs=5, pool=("fixed", 12), seed=4)
    wl = W.make_workload(spec)
    wl.q[:, 1] = wl.q[:, 0]
    out = run_oracle(wl)
    assert np.array_equal(out[:, 1], out[:, 0])
    assert not np.array_equal(out[:, 4], out[:, 0])


def test_shared_prefix_sequences_with_equal_queries_agree():
    spec = tiny_spec("bf16", "bf16", B=4, hq=4, hkv=2, D=64,
                     lens=("fixed", [100, 100, 40, 300]), mbs=19,
                     pool=("ratio", 1.2), prefix=128, seed=6)
    wl = W.make_workload(spec)
    assert np.array_equal(wl.block_table[0, :7], wl.block_table[1, :7])
    wl.q[1] = wl.q[0]
    out = run_oracle(wl)
    assert np.array_equal(out[0], out[1])


# ------------------------------------------- planted mistakes are caught

def _pins_pass(fn):
    """Run the brute-force and SDPA-style comparisons against `fn`."""
    spec = tiny_spec("f16", "f16", B=2, hq=4, hkv=2, D=16, lens=("fixed", [21, 40]),
                     mbs=3, pool=("fixed", 8), seed=21)
    wl = W.make_workload(spec)
    out = fn(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens, wl.scale,
             "f16", "f16")
    bout, _ = brute_decode(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens,
                           wl.scale, "f16", "f16")
    return np.allclose(out, bout, rtol=0, atol=1e-9)


def test_pins_catch_planted_mistakes(monkeypatch):
    import oracle.paged_decode as pd
    assert _pins_pass(pd.paged_decode_ref)

    real_gather = pd.gather_kv

    def swapped_kv_head(k, v, blocks, g, L, dt):
        return real_gather(k, v, blocks, (g + 1) % k.shape[1], L, dt)

    def transposed_v_page(k, v, blocks, g, L, dt):
        kr, _ = real_gather(k, v, blocks, g, L, dt)
        vp = pd.decode(v[blocks, g], dt)        # wrong: treats [D][16] as [16][D]
        vr = vp.reshape(len(blocks), 16, -1).reshape(len(blocks) * 16, -1)
        return kr, vr[:L]

    def off_by_one_length(k, v, blocks, g, L, dt):
        kr, vr = real_gather(k, v, blocks, g, min(L + 1, len(blocks) * 16), dt)
        return kr, vr

    real_attend = pd.attend

    def dropped_scale(q64, kr, vr, scale64):
        return real_attend(q64, kr, vr, 1.0)

    for name, fn in (("gather_kv", swapped_kv_head), ("gather_kv", transposed_v_page),
                     ("attend", dropped_scale)):
        monkeypatch.setattr(pd, name, fn)
        assert not _pins_pass(pd.paged_decode_ref), fn.__name__
        monkeypatch.undo()
    # reading one slot past the end reads a NaN-poisoned tail slot
    monkeypatch.setattr(pd, "gather_kv", off_by_one_length)
    spec = tiny_spec("f16", "f16", B=2, hq=4, hkv=2, D=16, lens=("fixed", [21, 40]),
                     mbs=3, pool=("fixed", 8), seed=21)
    wl = W.make_workload(spec)
    o = pd.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                            wl.context_lens, wl.scale, "f16", "f16")
    assert np.isnan(o).any()
