"""Pins for the multi-token query oracle (oracle/multi_query.py), CPU only:
torch's scaled-dot-product attention with its own causal mask over a full
square query block, the pure-Python brute force (tests/brute.py) run once per
new token on the visible prefix, closed forms for identical keys, and the
reductions to single-token decode (one new token; the last new token sees
the whole context)."""
import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_05_amd import workloads as W
from tests.brute import brute_decode
from tests.test_oracle_pins import DTYPES, explicit_gather, tiny_spec, torch_decode


def mq(wl, q, **kw):
    return oracle.multi_query_ref(q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens,
                                  wl.scale, wl.spec.io_dtype, wl.spec.kv_dtype, wl.k_scale,
                                  wl.v_scale, **kw)


@pytest.mark.parametrize("io,kv", DTYPES)
@pytest.mark.parametrize("T", [1, 3, 16])
def test_matches_torch_sdpa_with_its_causal_mask(io, kv, T):
    """Query row i of an L x L causal block sees keys 0 .. i (torch's own
    mask); the new tokens are its last T rows, the rows before them are
    filler. Rows of a sequence shorter than T have nothing to see."""
    spec = tiny_spec(io, kv, B=4, hq=8, hkv=2, D=32, lens=("fixed", [1, 9, 40, 130]),
                     mbs=9, pool=("fixed", 24), seed=6)
    wl = W.make_workload(spec)
    q = W.multi_query(wl, T)
    out, lse = mq(wl, q, return_lse=True)
    qd = torch_decode(q, io)                               # [B, T, Hq, D]
    fill = torch.randn((200, spec.num_q_heads, spec.head_dim), dtype=torch.float64,
                       generator=torch.Generator().manual_seed(1))
    for b in range(spec.batch):
        L = int(wl.context_lens[b])
        Ks, Vs = [], []
        for g in range(spec.num_kv_heads):
            K, V = explicit_gather(wl, b, g)
            K, V = torch_decode(K.numpy(), kv), torch_decode(V.numpy(), kv)
            if kv == "fp8_e4m3":
                K, V = K * float(wl.k_scale[g]), V * float(wl.v_scale[g])
            Ks.append(K)
            Vs.append(V)
        K, V = torch.stack(Ks)[None], torch.stack(Vs)[None]   # [1, Hkv, L, D]
        n_new = min(T, L)
        rows = torch.cat([fill[: L - n_new], qd[b, T - n_new:]])   # [L, Hq, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            rows.transpose(0, 1)[None], K, V, is_causal=True, scale=float(wl.scale),
            enable_gqa=True)[0].transpose(0, 1).numpy()          # [L, Hq, D]
        np.testing.assert_allclose(out[b, T - n_new:], ref[L - n_new:], rtol=0, atol=1e-12)
        assert (out[b, : T - n_new] == 0).all() and np.isneginf(lse[b, : T - n_new]).all()


@pytest.mark.parametrize("io,kv", [("f32", "f32"), ("bf16", "fp8_e4m3")])
def test_matches_brute_force_per_new_token(io, kv):
    spec = tiny_spec(io, kv, B=3, hq=4, hkv=2, D=16, lens=("fixed", [3, 16, 37]), seed=2)
    wl = W.make_workload(spec)
    T = 5
    q = W.multi_query(wl, T)
    out, lse = mq(wl, q, return_lse=True)
    for t in range(T):
        lens = np.maximum(wl.context_lens.astype(np.int64) - T + t + 1, 0)
        bout, blse = brute_decode(np.ascontiguousarray(q[:, t]), wl.k_cache, wl.v_cache,
                                  wl.block_table, lens, wl.scale, io, kv, wl.k_scale,
                                  wl.v_scale)
        np.testing.assert_allclose(out[:, t], bout, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(lse[:, t]), np.isneginf(blse))
        fin = np.isfinite(blse)
        np.testing.assert_allclose(lse[:, t][fin], blse[fin], rtol=0, atol=1e-12)


def test_one_new_token_is_decode_and_the_last_sees_everything():
    spec = tiny_spec("f16", "f16", B=4, hq=8, hkv=2, D=64, lens=("fixed", [1, 17, 100, 256]),
                     mbs=16, pool=("fixed", 40), seed=9)
    wl = W.make_workload(spec)
    q1 = W.multi_query(wl, 1)
    out1, lse1 = mq(wl, q1, return_lse=True)
    ref1, rlse1 = oracle.paged_decode_ref(np.ascontiguousarray(q1[:, 0]), wl.k_cache, wl.v_cache,
                                          wl.block_table, wl.context_lens, wl.scale, "f16",
                                          "f16", return_lse=True)
    assert np.array_equal(out1[:, 0], ref1) and np.array_equal(lse1[:, 0], rlse1)
    q8 = W.multi_query(wl, 8)
    out8 = mq(wl, q8)
    ref8 = oracle.paged_decode_ref(np.ascontiguousarray(q8[:, 7]), wl.k_cache, wl.v_cache,
                                   wl.block_table, wl.context_lens, wl.scale, "f16", "f16")
    assert np.array_equal(out8[:, 7], ref8)


@pytest.mark.parametrize("L,T", [(40, 16), (16, 16), (5, 8), (300, 7)])
def test_identical_keys_average_the_visible_values(L, T):
    """All keys equal: every visible token weighs the same, so new token t
    returns the mean of V rows 0 .. L-T+t and lse = s + ln(L-T+t+1). A
    visible count off by one changes every row."""
    spec = tiny_spec("f32", "f32", B=1, hq=2, hkv=1, D=16, lens=("fixed", [L]),
                     mbs=-(-L // 16), pool=("fixed", -(-L // 16) + 2), seed=4)
    wl = W.make_workload(spec, poison=False)
    wl.k_cache[:] = wl.k_cache[:1, :, :, :1, :]            # one key row everywhere
    q = W.multi_query(wl, T)
    out, lse = mq(wl, q, return_lse=True)
    K, V = explicit_gather(wl, 0, 0)
    K, V = K.numpy().astype(np.float64), V.numpy().astype(np.float64)
    sc = float(wl.scale)
    for t in range(T):
        n = L - T + t + 1
        for h in range(2):
            if n <= 0:
                assert (out[0, t, h] == 0).all() and lse[0, t, h] == -math.inf
                continue
            np.testing.assert_allclose(out[0, t, h], V[:n].mean(axis=0), rtol=0, atol=1e-12)
            s = sc * float(q[0, t, h].astype(np.float64) @ K[0])
            assert abs(lse[0, t, h] - (s + math.log(n))) < 1e-12
            if n > 1:
                assert not np.allclose(out[0, t, h], V[: n - 1].mean(axis=0), rtol=0, atol=1e-9)


def _mutated_multi(kind):
    """The oracle's definition with one plausible mistake planted."""
    from oracle.formats import decode
    from oracle.paged_decode import attend, gather_kv

    def fn(q, k_cache, v_cache, block_table, context_lens, scale, io, kv):
        qv = decode(q, io)
        B, T, Hq, D = qv.shape
        if kind == "layout":                       # q read as [B][Hq][T][D]
            qv = qv.reshape(B, Hq, T, D).transpose(0, 2, 1, 3)
        Hkv = k_cache.shape[1]
        G = Hq // Hkv
        out = np.zeros((B, T, Hq, D))
        for b in range(B):
            L = int(context_lens[b])
            blocks = np.asarray(block_table[b, : -(-L // 16)], dtype=np.int64)
            for g in range(Hkv):
                kr, vr = gather_kv(k_cache, v_cache, blocks, g, L, kv)
                for t in range(T):
                    n = {"offset": L - T + t, "nocausal": L}.get(kind, L - T + t + 1)
                    tq = T - 1 - t if kind == "reverse" else t
                    n = max(n, 0)
                    o, _ = attend(qv[b, tq, g * G:(g + 1) * G], kr[:n], vr[:n],
                                  float(np.float32(scale)))
                    out[b, t, g * G:(g + 1) * G] = o
        return out
    return fn


@pytest.mark.parametrize("kind", ["offset", "nocausal", "reverse", "layout"])
def test_pins_catch_planted_mistakes(kind):
    spec = tiny_spec("f32", "f32", B=3, hq=4, hkv=2, D=16, lens=("fixed", [6, 16, 37]), seed=2)
    wl = W.make_workload(spec)
    T = 5
    q = W.multi_query(wl, T)
    args = (q, wl.k_cache, wl.v_cache, wl.block_table, wl.context_lens, wl.scale, "f32", "f32")
    good = mq(wl, q)
    brute = np.stack([brute_decode(np.ascontiguousarray(q[:, t]), wl.k_cache, wl.v_cache,
                                   wl.block_table,
                                   np.maximum(wl.context_lens.astype(np.int64) - T + t + 1, 0),
                                   wl.scale, "f32", "f32")[0] for t in range(T)], axis=1)
    np.testing.assert_allclose(good, brute, rtol=0, atol=1e-12)
    bad = _mutated_multi(kind)(*args)
    assert not np.allclose(bad, brute, rtol=0, atol=1e-6), kind
