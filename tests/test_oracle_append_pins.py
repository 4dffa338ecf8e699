"""Pins for the KV-append oracle (oracle/kv_append.py): the E4M3 encoder
against torch's float8_e4m3fn cast, the exhaustive code round trip and hand
worked ties; the append against a flat-offset brute force and the decode
oracle. CPU only."""
import struct

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_05_amd import workloads as W


# ------------------------------------------------------------------ encoder

def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.E4M3_TABLE[codes]
    vals[codes == 0x80] = -0.0
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_encoder_matches_torch_cast_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (0.01, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448.0, 448.0).astype(np.float32)
    # every midpoint between neighbouring codes, and its float32 neighbours
    pos = oracle.E4M3_TABLE[:127]
    mid = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    near = np.concatenate([mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))])
    x = np.concatenate([x, near, -near, np.float32([0.0, -0.0, 1e-30, -1e-30])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.e4m3_encode(x)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38),      # half-way 1.0 (0x38) .. 1.125 (0x39): even code 0x38
    (1.1875, 0x3A),      # half-way 1.125 (0x39) .. 1.25 (0x3A): even code 0x3A
    (2.0 ** -10, 0x00),  # half the least subnormal: ties to 0
    (3 * 2.0 ** -10, 0x02),   # half-way 2^-9 (0x01) .. 2^-8 (0x02)
    (432.0, 0x7E),       # half-way 416 (0x7D) .. 448 (0x7E): even code 0x7E
    (500.0, 0x7E), (1e30, 0x7E), (float("inf"), 0x7E),   # clamped to 448
    (-500.0, 0xFE), (float("-inf"), 0xFE),
    (float("nan"), 0x7F), (-0.0, 0x80), (-1e-30, 0x80),
])
def test_encoder_hand_worked(value, code):
    assert int(oracle.e4m3_encode(np.float64(value).reshape(1))[0]) == code


def test_quantize_divides_in_float32():
    # the division is a float32 one: 1/3 is first rounded to float32
    raw = np.float32([1.0]).view(np.float32)
    got = oracle.quantize_e4m3(raw, "f32", np.float32(3.0))
    want = oracle.e4m3_encode(np.float32(1.0) / np.float32(3.0))
    assert np.array_equal(got, want.reshape(1))
    # and matches the generator's quantizer (clamp, then torch's cast)
    rng = np.random.default_rng(2)
    x = rng.standard_normal(5000).astype(np.float32)
    scale = np.float32(np.abs(x).max() / 448.0)
    ours = oracle.quantize_e4m3(x, "f32", scale)
    ref = torch.from_numpy(np.clip(x / scale, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------- append

def _flat_brute(k_cache, v_cache, k_new, v_new, bt, pos, src, kv, ks, vs):
    """The append by flat byte offsets into the raw cache buffers."""
    kb = bytearray(np.ascontiguousarray(k_cache).tobytes())
    vb = bytearray(np.ascontiguousarray(v_cache).tobytes())
    nb, H = k_cache.shape[:2]
    D = k_new.shape[2]
    eb = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}[kv]
    X = 16 // eb
    page = 16 * D * eb
    for b in range(k_new.shape[0]):
        p = int(pos[b])
        if not 0 <= p < 16 * bt.shape[1]:
            continue
        blk = int(bt[b, p // 16])
        if not 0 <= blk < nb:
            continue
        for g in range(H):
            base = (blk * H + g) * page
            for d in range(D):
                for arr, buf, scale, off in (
                        (k_new, kb, ks, base + ((d // X) * 16 * X + (p % 16) * X + d % X) * eb),
                        (v_new, vb, vs, base + (d * 16 + p % 16) * eb)):
                    if kv == src:
                        word = np.ascontiguousarray(arr[b, g, d:d + 1]).tobytes()
                    else:
                        x = float(oracle.decode(arr[b, g, d:d + 1], src)[0])
                        y = struct.unpack("f", struct.pack("f", np.float32(x) / np.float32(scale[g])))[0]
                        word = bytes([int(oracle.e4m3_encode(np.float64(y).reshape(1))[0])])
                    buf[off:off + eb] = word
    kc = np.frombuffer(bytes(kb), dtype=k_cache.dtype).reshape(k_cache.shape)
    vc = np.frombuffer(bytes(vb), dtype=v_cache.dtype).reshape(v_cache.shape)
    return kc, vc


def _append_case(src, kv, D=16, B=4, H=2, seed=3):
    spec = W.Spec(f"app_{src}_{kv}", B, 2 * H, H, D, src, kv, ("fixed", [3, 16, 17, 40][:B]),
                  4, ("fixed", 14), 0, 0, seed)
    wl = W.make_workload(spec, poison=False)
    rng = np.random.default_rng(seed + 100)
    new = rng.standard_normal((2, B, H, D)).astype(np.float32) * 3
    from paged_kv_decode_05_amd.workloads import _to_storage   # storage rounding of the generator
    k_new, v_new = _to_storage(new[0], src), _to_storage(new[1], src)
    return wl, k_new, v_new


@pytest.mark.parametrize("src,kv", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                    ("f16", "fp8_e4m3"), ("bf16", "fp8_e4m3"), ("f32", "fp8_e4m3")])
def test_append_matches_flat_offset_brute_force(src, kv):
    wl, k_new, v_new = _append_case(src, kv)
    pos = np.array([3, 15, 70, -1], dtype=np.int32)    # 70 lies past the table, -1 is padding
    ks = wl.k_scale if kv == "fp8_e4m3" else None
    vs = wl.v_scale if kv == "fp8_e4m3" else None
    if kv == "fp8_e4m3" and ks is None:
        ks = vs = np.float32([0.05, 0.07])
    got = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new, wl.block_table, pos, src, kv, ks, vs)
    want = _flat_brute(wl.k_cache, wl.v_cache, k_new, v_new, wl.block_table, pos, src, kv, ks, vs)
    assert np.array_equal(got[0].view(np.uint8), want[0].view(np.uint8))
    assert np.array_equal(got[1].view(np.uint8), want[1].view(np.uint8))


def test_append_touches_only_the_target_slots_and_skips_bad_entries():
    wl, k_new, v_new = _append_case("f16", "f16")
    bt = wl.block_table.copy()
    bt[2, 1] = wl.num_blocks + 5                     # block id outside the pool
    pos = np.array([5, -3, 17, 64], dtype=np.int32)   # only sequence 0 is written
    k2, v2 = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new, bt, pos, "f16", "f16")
    blk = int(bt[0, 0])
    dk = np.argwhere(k2.view(np.uint16) != wl.k_cache.view(np.uint16))
    dv = np.argwhere(v2.view(np.uint16) != wl.v_cache.view(np.uint16))
    assert set(dk[:, 0]) <= {blk} and set(dk[:, 3]) <= {5}
    assert set(dv[:, 0]) <= {blk} and set(dv[:, 3]) <= {5}
    assert len(dk) > 0 and len(dv) > 0


@pytest.mark.parametrize("src,kv", [("f16", "f16"), ("bf16", "fp8_e4m3")])
def test_appended_row_is_what_decode_then_reads(src, kv):
    # Append at position L (the next free slot), grow the context to L + 1 and
    # decode: the result equals attention over the old rows plus the new one.
    wl, k_new, v_new = _append_case(src, kv)
    ks = wl.k_scale if kv == "fp8_e4m3" else None
    vs = wl.v_scale if kv == "fp8_e4m3" else None
    L = wl.context_lens.astype(np.int32)
    k2, v2 = oracle.kv_append_ref(wl.k_cache, wl.v_cache, k_new, v_new, wl.block_table, L, src, kv, ks, vs)
    out = oracle.paged_decode_ref(wl.q, k2, v2, wl.block_table, L + 1, wl.scale, src, kv, ks, vs)
    H, D = k_new.shape[1:]
    G = wl.q.shape[1] // H
    for b in range(len(L)):
        blocks = wl.block_table[b, : -(-int(L[b] + 1) // 16)]
        for g in range(H):
            kr, vr = oracle.gather_kv(k2, v2, blocks, g, int(L[b]) + 1, kv)
            if kv == "fp8_e4m3":
                kr, vr = kr * float(ks[g]), vr * float(vs[g])
                kn = oracle.E4M3_TABLE[oracle.quantize_e4m3(k_new[b, g], src, ks[g])] * float(ks[g])
            else:
                kn = oracle.decode(k_new[b, g], src)
            assert np.array_equal(kr[-1], kn)
            q = oracle.decode(wl.q[b, g * G:(g + 1) * G], src)
            o, _ = oracle.attend(q, kr, vr, float(np.float32(wl.scale)))
            assert np.allclose(out[b, g * G:(g + 1) * G], o, rtol=1e-12, atol=1e-12)
