"""The C ABI without a GPU: the library loads, exports every function the
header declares, validates arguments on the host, and sizes workspaces."""
import ctypes
import os
import re

import pytest

import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "padecode.h")

pytestmark = pytest.mark.skipif(not os.path.exists(pkd.library_path()),
                                reason="libpadecode.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_bound_functions():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pkd.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def shape(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                max_blocks_per_seq=32, num_blocks=100, partition_size=0)
    base.update(kw)
    return _lib.PaShape(**base)


FAKE = 1 << 20      # a 16-byte-aligned non-null pointer value; never dereferenced


def call(s, io=1, kv=1, ks=None, vs=None, ws=None, wsb=0, out=FAKE, q=FAKE, k=FAKE,
         v=FAKE, bt=FAKE, cl=FAKE, lse=None):
    lib = _lib.load_library()
    sp = ctypes.byref(s) if s is not None else None
    return lib.pa_decode(sp, q, k, v, bt, cl, 0.1, io, kv, ks, vs, ws, wsb, out, lse, None)


def test_null_arguments_are_rejected_before_any_launch():
    assert call(None) == 1
    for kw in ("q", "k", "v", "bt", "cl", "out"):
        assert call(shape(), **{kw: None}) == 1, kw
    assert call(shape(), io=1, kv=3) == 1            # fp8 without scales


@pytest.mark.parametrize("bad", [
    dict(num_q_heads=7), dict(num_q_heads=40, num_kv_heads=2), dict(head_dim=96),
    dict(head_dim=256), dict(block_size=32), dict(partition_size=24),
    dict(partition_size=-16), dict(max_blocks_per_seq=0), dict(num_blocks=0),
    dict(batch=-1), dict(num_kv_heads=0), dict(batch=70000), dict(partition_size=-2),
    # balanced split: batch beyond the workgroup-wide scan, line beyond int32
    dict(partition_size=-1, batch=4097),
    dict(partition_size=-1, batch=4096, num_q_heads=64, num_kv_heads=64,
         max_blocks_per_seq=1 << 13)])
def test_unsupported_shapes_are_errors(bad):
    assert call(shape(**bad)) == 2


def test_dtype_rules():
    assert call(shape(), io=0, kv=3, ks=FAKE, vs=FAKE) == 3   # fp8 cache needs 16-bit io
    assert call(shape(), io=1, kv=2) == 3
    assert call(shape(), io=3, kv=3, ks=FAKE, vs=FAKE) == 3
    assert call(shape(), io=7, kv=7) == 3


def test_alignment_rules():
    assert call(shape(), q=FAKE + 8) == 5
    assert call(shape(), out=FAKE + 2) == 5
    assert call(shape(), bt=FAKE + 2) == 5


def test_workspace_rules():
    s = shape(partition_size=512)
    need = _lib.load_library().pa_decode_workspace_bytes(ctypes.byref(s))
    assert call(s) == 4
    assert call(s, ws=FAKE, wsb=need - 1) == 4
    assert call(s, ws=FAKE + 16, wsb=need) == 5      # workspace must be 256-byte aligned
    assert call(shape(batch=0, partition_size=512), ws=FAKE, wsb=need) == 0  # empty batch: no-op


def test_workspace_size_arithmetic():
    lib = _lib.load_library()

    def ws(**kw):
        return lib.pa_decode_workspace_bytes(ctypes.byref(shape(**kw)))

    def up(x):
        return (x + 255) // 256 * 256

    assert ws() == 0
    # B=32, Hq=28, Hkv=4, D=128, MBS=256, partition 512 -> 8 partitions
    b, hq, hkv, d, p = 32, 28, 4, 128, 8
    expect = up(b * hq * p * d * 4) + up(b * hq * p * 4) + up(b * hkv * 4)
    assert ws(batch=b, num_q_heads=hq, num_kv_heads=hkv, max_blocks_per_seq=256,
              partition_size=512) == expect
    # partitions round up: MBS*16 = 512 tokens / 48 -> 11
    expect = up(2 * 8 * 11 * 128 * 4) + up(2 * 8 * 11 * 4) + up(2 * 2 * 4)
    assert ws(partition_size=48) == expect
    # more than 16 partitions per sequence: a second merge level. 32
    # partitions of 16 tokens -> groups of F = 16, 2 group pieces per
    # (sequence, query head) after the partition pieces, 2 more counters per
    # (sequence, KV head)
    rows = 2 * 2 * (32 + 2) * 4
    assert ws(partition_size=16) == up(2 * 2 * 3 * 4) + up(rows * 128 * 4) + up(rows * 4)
    # 16 partitions: one level
    rows = 2 * 2 * 16 * 4
    assert ws(partition_size=32) == up(2 * 2 * 4) + up(rows * 128 * 4) + up(rows * 4)
    # 8192 partitions: F = 91 (90 * 90 < 8192 <= 91 * 91), 91 groups
    rows = 1 * 1 * (8192 + 91) * 8
    assert ws(batch=1, num_q_heads=8, num_kv_heads=1, max_blocks_per_seq=8192,
              partition_size=16) == up(1 * 1 * 92 * 4) + up(rows * 128 * 4) + up(rows * 4)
    assert lib.pa_decode_workspace_bytes(None) == 0
    assert ws(head_dim=100) == 0


def test_status_strings():
    lib = _lib.load_library()
    for code in range(10):
        assert lib.pa_status_str(code) and lib.pa_status_str(code) != b"unknown status"
    assert lib.pa_status_str(99) == b"unknown status"


def test_balanced_split_shapes_pass_validation():
    # Valid balanced shapes pass validation; without a GPU the call stops at
    # the device query (PA_ERR_HIP, nothing launched) and the workspace size
    # is unknown (0). Where a GPU is present this call would launch on the
    # fake pointers, so it is left to the GPU tests.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: valid shapes would launch")
    lib = _lib.load_library()
    for kw in (dict(batch=4096), dict(batch=1, max_blocks_per_seq=8192),
               dict(batch=32, num_q_heads=28, num_kv_heads=4, max_blocks_per_seq=256)):
        s = shape(partition_size=-1, **kw)
        assert call(s, ws=FAKE, wsb=1 << 30) == 6, kw
        assert lib.pa_decode_workspace_bytes(ctypes.byref(s)) == 0


def call_append(s, src=1, kv=1, ks=None, vs=None, kn=FAKE, vn=FAKE, pos=FAKE, bt=FAKE,
                kc=FAKE, vc=FAKE):
    lib = _lib.load_library()
    sp = ctypes.byref(s) if s is not None else None
    return lib.pa_kv_append(sp, kn, vn, pos, bt, src, kv, ks, vs, kc, vc, None)


def test_append_rejects_bad_arguments_before_any_launch():
    assert call_append(None) == 1
    for kw in ("kn", "vn", "pos", "bt", "kc", "vc"):
        assert call_append(shape(), **{kw: None}) == 1, kw
    assert call_append(shape(), src=1, kv=3) == 1                  # fp8 without scales
    assert call_append(shape(head_dim=96)) == 2
    assert call_append(shape(block_size=8)) == 2
    assert call_append(shape(num_kv_heads=0)) == 2
    assert call_append(shape(max_blocks_per_seq=0)) == 2
    assert call_append(shape(), src=1, kv=2) == 3                  # f16 rows into a bf16 cache
    assert call_append(shape(), src=3, kv=3, ks=FAKE, vs=FAKE) == 3   # fp8 rows
    assert call_append(shape(), kn=FAKE + 1) == 5
    assert call_append(shape(), kc=FAKE + 8) == 5
    assert call_append(shape(), pos=FAKE + 2) == 5
    assert call_append(shape(batch=0)) == 0                         # empty batch: no-op


def test_lse_merge_rejects_bad_arguments_before_any_launch():
    lib = _lib.load_library()
    m = lib.pa_lse_merge
    assert m(0, 4, 128, FAKE, FAKE, 1, FAKE, None, None) == 2        # no shards
    assert m(2, -1, 128, FAKE, FAKE, 1, FAKE, None, None) == 2
    assert m(2, 4, 6, FAKE, FAKE, 1, FAKE, None, None) == 2          # head_dim % 4
    assert m(2, 4, 2048, FAKE, FAKE, 1, FAKE, None, None) == 2
    assert m(2, 4, 128, None, FAKE, 1, FAKE, None, None) == 1
    assert m(2, 4, 128, FAKE, None, 1, FAKE, None, None) == 1
    assert m(2, 4, 128, FAKE, FAKE, 1, None, None, None) == 1
    assert m(2, 4, 128, FAKE, FAKE, 3, FAKE, None, None) == 3        # fp8 outputs
    assert m(2, 4, 128, FAKE + 8, FAKE, 1, FAKE, None, None) == 5
    assert m(2, 4, 128, FAKE, FAKE + 2, 1, FAKE, None, None) == 5
    assert m(2, 0, 128, FAKE, FAKE, 1, FAKE, None, None) == 0        # no rows: no-op


def call_multi(s, q_len=4, io=1, kv=1, ks=None, vs=None, ws=None, wsb=0, out=FAKE, q=FAKE,
               k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, lse=None):
    lib = _lib.load_library()
    sp = ctypes.byref(s) if s is not None else None
    return lib.pa_decode_multi(sp, q_len, q, k, v, bt, cl, 0.1, io, kv, ks, vs, ws, wsb, out,
                               lse, None)


def test_multi_token_call_rejects_bad_arguments_before_any_launch():
    assert call_multi(None) == 1
    for kw in ("q", "k", "v", "bt", "cl", "out"):
        assert call_multi(shape(), **{kw: None}) == 1, kw
    for T in (0, 17, -1):
        assert call_multi(shape(), q_len=T) == 2
    assert call_multi(shape(partition_size=24)) == 2
    assert call_multi(shape(num_q_heads=40, num_kv_heads=2)) == 2
    assert call_multi(shape(), io=0, kv=3, ks=FAKE, vs=FAKE) == 3
    assert call_multi(shape(), io=1, kv=3) == 1
    assert call_multi(shape(), q=FAKE + 8) == 5
    s = shape(partition_size=512)
    need = _lib.load_library().pa_decode_multi_workspace_bytes(ctypes.byref(s), 4)
    assert call_multi(s) == 4
    assert call_multi(s, ws=FAKE, wsb=need - 1) == 4
    assert call_multi(s, ws=FAKE + 16, wsb=need) == 5
    assert call_multi(shape(batch=0, partition_size=512), ws=FAKE, wsb=need) == 0


def test_multi_token_balanced_split_of_wide_rows_passes_validation():
    # 20 rows (wider than one tile) take the wide-row balanced split; without
    # a GPU the call stops at the device query (PA_ERR_HIP, nothing launched)
    # and the workspace size is unknown (0). With a GPU present this call
    # would launch on the fake pointers, so it is left to the GPU tests.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: valid shapes would launch")
    lib = _lib.load_library()
    s = shape(partition_size=-1)
    assert call_multi(s, q_len=5, ws=FAKE, wsb=1 << 30) == 6
    assert lib.pa_decode_multi_workspace_bytes(ctypes.byref(s), 5) == 0
    assert call_multi(shape(partition_size=-1, batch=4097), q_len=5) == 2     # beyond the scan
    assert call_multi(shape(partition_size=-2), q_len=5) == 2


def call_prefix(s, prefix_blocks, io=1, kv=1, ws=None, wsb=0, q=FAKE, out=FAKE, bt=FAKE):
    lib = _lib.load_library()
    sp = ctypes.byref(s) if s is not None else None
    return lib.pa_decode_prefix(sp, prefix_blocks, q, FAKE, FAKE, bt, FAKE, 0.1, io, kv, None, None,
                                ws, wsb, out, None, None)


def test_shared_prefix_call_validates_before_the_device_query():
    bal = dict(partition_size=-1)
    assert call_prefix(None, 4) == 1
    assert call_prefix(shape(**bal), -1) == 2
    assert call_prefix(shape(**bal), 33) == 2                   # beyond max_blocks_per_seq
    assert call_prefix(shape(partition_size=0), 4) == 2         # balanced split only
    assert call_prefix(shape(partition_size=512), 4) == 2
    assert call_prefix(shape(partition_size=-1, batch=4097), 4) == 2
    assert call_prefix(shape(partition_size=-1, head_dim=96), 4) == 2
    assert call_prefix(shape(**bal), 4, q=None) == 1
    assert call_prefix(shape(**bal), 4, bt=None) == 1
    assert call_prefix(shape(**bal), 4, io=0, kv=3) == 3        # f32 q with an fp8 cache
    lib = _lib.load_library()
    assert lib.pa_decode_prefix_workspace_bytes(ctypes.byref(shape(partition_size=512))) == 0
    assert lib.pa_decode_prefix_workspace_bytes(None) == 0


def test_shared_prefix_call_passes_validation():
    # Without a GPU a valid call stops at the device query (PA_ERR_HIP,
    # nothing launched) and the workspace size is unknown (0); with a GPU it
    # would launch on the fake pointers, so it is left to the GPU tests.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: valid shapes would launch")
    lib = _lib.load_library()
    s = shape(partition_size=-1)
    assert call_prefix(s, 0, ws=FAKE, wsb=1 << 30) == 6
    assert call_prefix(s, 32, ws=FAKE, wsb=1 << 30) == 6
    assert lib.pa_decode_prefix_workspace_bytes(ctypes.byref(s)) == 0


def test_multi_token_workspace_size_arithmetic():
    lib = _lib.load_library()

    def ws(T, **kw):
        return lib.pa_decode_multi_workspace_bytes(ctypes.byref(shape(**kw)), T)

    def up(x):
        return (x + 255) // 256 * 256

    assert ws(4) == 0 and ws(0, partition_size=512) == 0 and ws(17, partition_size=512) == 0
    assert lib.pa_decode_multi_workspace_bytes(None, 4) == 0
    # B=32, Hq=28, Hkv=4 (G=7), T=8 -> 56 rows = 4 column tiles = 2 chunks;
    # MBS=256, partition 512 -> 8 partitions
    b, hkv, d, p, rows, chunks = 32, 4, 128, 8, 56, 2
    expect = up(b * hkv * chunks * 4) + up(b * hkv * p * rows * d * 4) + up(b * hkv * p * rows * 4)
    assert ws(8, batch=b, num_q_heads=28, num_kv_heads=hkv, max_blocks_per_seq=256,
              partition_size=512) == expect
    # G=16, T=16: 256 rows, 8 chunks; one partition of 16 tokens per block:
    # 32 partitions, so two merge levels with groups of 16 (2 group slots
    # after the 32 partition slots, 2 more counters per chunk)
    expect = up(2 * 1 * 3 * 8 * 4) + up(2 * 1 * 34 * 256 * 64 * 4) + up(2 * 1 * 34 * 256 * 4)
    assert ws(16, batch=2, num_q_heads=16, num_kv_heads=1, head_dim=64,
              partition_size=16) == expect
    # one new token: the same rows as decode, one counter per (sequence, KV head)
    s = shape(partition_size=512)
    assert ws(1, partition_size=512) == lib.pa_decode_workspace_bytes(ctypes.byref(s))


def test_multi_token_rows_of_one_tile_take_the_decode_kernels():
    # G * q_len <= 16: the decode kernels' workspace layout (one counter per
    # (sequence, KV head)) and the balanced split are available
    lib = _lib.load_library()
    s = shape(partition_size=512)                 # G = 4
    rows4 = lib.pa_decode_multi_workspace_bytes(ctypes.byref(s), 4)
    up = lambda x: (x + 255) // 256 * 256
    b, hkv, p, d, rows = 2, 2, 32, 128, 16        # 32 blocks of 16 tokens / 512 = 1 partition
    p = (32 * 16 + 511) // 512
    assert rows4 == up(b * hkv * 4) + up(b * hkv * p * rows * d * 4) + up(b * hkv * p * rows * 4)
    if torch_gpu_count() == 0:                    # stops at the device query, nothing launched
        assert call_multi(shape(partition_size=-1), q_len=4) == 6


def torch_gpu_count():
    import torch
    return torch.cuda.device_count()


def call_noalloc(s, io=1, kv=1, ks=None, vs=None, out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE,
                 cl=FAKE, lse=None):
    lib = _lib.load_library()
    sp = ctypes.byref(s) if s is not None else None
    return lib.pa_decode_noalloc(sp, q, k, v, bt, cl, 0.1, io, kv, ks, vs, out, lse, None)


def test_noalloc_rejects_calls_beyond_its_scratch_before_any_launch():
    assert call_noalloc(None) == 1
    # 512-token partitions, 28/4 heads, 4096-token tables: partial results of
    # 8 partitions x 7 rows x 129 floats per (sequence, KV head) pair; 16 MiB
    # minus the 256 KiB counter region holds about 570 pairs, not 2400
    big = shape(batch=600, num_q_heads=28, num_kv_heads=4, max_blocks_per_seq=256,
                partition_size=512)
    assert call_noalloc(big) == 9
    # more counters than the counter region holds (16 partitions of 16
    # tokens per sequence: one counter per pair, tiny partial results)
    many = shape(batch=65535, num_q_heads=2, num_kv_heads=2, head_dim=64, max_blocks_per_seq=1,
                 partition_size=16)
    assert call_noalloc(many) == 9
    for kw in ("q", "k", "v", "bt", "cl", "out"):       # argument checks as pa_decode
        assert call_noalloc(shape(), **{kw: None}) == 1, kw
    assert call_noalloc(shape(head_dim=96)) == 2
    assert call_noalloc(shape(), io=1, kv=2) == 3
    assert call_noalloc(shape(), q=FAKE + 8) == 5
    assert call_noalloc(shape(batch=0)) == 0


# ---- the binding's buffer checks, exercised on CPU tensors ------------------

def _buffers(dtype="f16", fp8=False):
    import torch
    tq = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    B, Hq, Hkv, D = 2, 8, 2, 128
    q = torch.zeros(B, Hq, D, dtype=tq)
    kd = torch.uint8 if fp8 else tq
    x = 16 if fp8 else 8
    k = torch.zeros(10, Hkv, D // x, 16, x, dtype=kd)
    v = torch.zeros(10, Hkv, D, 16, dtype=kd)
    bt = torch.zeros(B, 4, dtype=torch.int32)
    cl = torch.zeros(B, dtype=torch.int32)
    return q, (k, v, bt, cl)


def _check(q, inputs, **kw):
    return _lib.check_buffers(q, inputs, on_device=lambda t: True, **kw)


def test_buffer_checks_accept_well_formed_buffers():
    import torch
    q, inp = _buffers()
    _check(q, inp, out=torch.empty_like(q), lse_out=torch.empty(2, 8),
           workspace=torch.empty(1024, dtype=torch.uint8))
    q, inp = _buffers(fp8=True)
    _check(q, inp, k_scale=torch.ones(2), v_scale=torch.ones(2), fp8=True)


@pytest.mark.parametrize("what,status", [
    ("out_dtype", 3), ("out_shape", 2), ("out_strided", 2), ("lse_dtype", 3), ("lse_shape", 2),
    ("scale_dtype", 3), ("scale_shape", 2), ("scale_missing", 1), ("ws_dtype", 3),
    ("ws_strided", 2), ("host_out", 2), ("host_ws", 2), ("host_scale", 2)])
def test_buffer_checks_reject_misfit_buffers(what, status):
    import torch
    q, inp = _buffers(fp8=what.startswith("scale") or what == "host_scale")
    fp8 = q is not None and inp[0].dtype == torch.uint8
    kw = dict(k_scale=torch.ones(2), v_scale=torch.ones(2)) if fp8 else {}
    on_device = lambda t: True
    if what == "out_dtype":
        kw["out"] = torch.empty(q.shape, dtype=torch.float32)      # twice q's element size
    elif what == "out_shape":
        kw["out"] = torch.empty(2, 8, 64, dtype=q.dtype)
    elif what == "out_strided":
        kw["out"] = torch.empty(2, 8, 256, dtype=q.dtype)[..., ::2]
    elif what == "lse_dtype":
        kw["lse_out"] = torch.empty(2, 8, dtype=torch.bfloat16)
    elif what == "lse_shape":
        kw["lse_out"] = torch.empty(2, 4)
    elif what == "scale_dtype":
        kw["k_scale"] = torch.ones(2, dtype=torch.float16)
    elif what == "scale_shape":
        kw["v_scale"] = torch.ones(4)
    elif what == "scale_missing":
        kw.pop("k_scale")
    elif what == "ws_dtype":
        kw["workspace"] = torch.empty(256, dtype=torch.int32)
    elif what == "ws_strided":
        kw["workspace"] = torch.empty(512, dtype=torch.uint8)[::2]
    elif what.startswith("host_"):
        # the tensor named is the one that is not device memory
        target = {"host_out": "out", "host_ws": "workspace", "host_scale": "k_scale"}[what]
        kw.setdefault("out", torch.empty_like(q))
        kw.setdefault("workspace", torch.empty(256, dtype=torch.uint8))
        if target == "k_scale":
            kw["k_scale"] = torch.ones(2)
        bad = kw[target]
        on_device = lambda t: t is not bad
    with pytest.raises(_lib.PaError) as e:
        _lib.check_buffers(q, inp, on_device=on_device, fp8=fp8, **kw)
    assert e.value.status == status, (what, str(e.value))


@pytest.mark.parametrize("pb", [2**31, 2**32 + 5, -2**31 - 1])
def test_shared_prefix_count_outside_32_bits_is_refused_by_the_binding(pb):
    # the C ABI takes an int32: a wider value must not wrap into a valid one
    import torch
    q = torch.zeros(2, 8, 128, dtype=torch.float16)
    k = torch.zeros(4, 2, 16, 16, 8, dtype=torch.float16)
    v = torch.zeros(4, 2, 128, 16, dtype=torch.float16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    cl = torch.ones(2, dtype=torch.int32)
    with pytest.raises(_lib.PaError) as e:
        _lib.prepare(q, k, v, bt, cl, 0.1, partition_size=_lib.SPLIT_BALANCED, prefix_blocks=pb)
    assert e.value.status == 2 and "32-bit" in str(e.value)


def test_partition_size_outside_32_bits_is_refused_not_wrapped():
    # 2**32 + 512 would wrap to a valid 512-token split in the int32 field
    import torch
    q = torch.zeros(2, 8, 128, dtype=torch.float16)
    k = torch.zeros(4, 2, 16, 16, 8, dtype=torch.float16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    with pytest.raises(_lib.PaError) as e:
        _lib.make_shape(q, k, bt, 2**32 + 512)
    assert e.value.status == 2 and "partition_size" in str(e.value)
    assert _lib.make_shape(q, k, bt, 512).partition_size == 512
