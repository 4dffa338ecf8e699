"""ctypes binding to libpadecode.so (C ABI in include/padecode.h).

Argument marshalling only: shapes and dtypes are read off torch tensors and
passed as plain pointers; every step of the computation runs in the HIP
kernels. There is no fallback: if the library is missing, `decode` raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libpadecode.so"

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
SPLIT_BALANCED = -1   # partition_size value of the balanced split (PA_SPLIT_BALANCED)
DTYPE_CODE = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "fp8_e4m3": PA_FP8_E4M3}

EXPORTED = ("pa_decode", "pa_decode_workspace_bytes", "pa_decode_noalloc", "pa_decode_multi",
            "pa_decode_multi_workspace_bytes", "pa_decode_prefix", "pa_decode_prefix_workspace_bytes",
            "pa_kv_append", "pa_lse_merge",
            "pa_workspace_reset", "pa_status_str", "pa_pool_create", "pa_pool_destroy",
            "pa_pool_add_sequence", "pa_pool_append_token", "pa_pool_free_sequence",
            "pa_pool_num_free", "pa_pool_block_table", "pa_pool_shared_prefix")
PA_ERR_CAPACITY, PA_ERR_STATE, PA_ERR_SCRATCH = 7, 8, 9
NOALLOC_SCRATCH_BYTES = 16 << 20    # PA_NOALLOC_SCRATCH_BYTES
NOALLOC_COUNTER_BYTES = 256 << 10   # PA_NOALLOC_COUNTER_BYTES


class PaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"pa_decode failed ({status}): {msg}")
        self.status = status


def _c_int(x, bits, what):
    """x as an int that fits a signed `bits`-bit C argument (ctypes would
    wrap a wider value into one the library might accept)."""
    v = int(x)
    if not -(1 << (bits - 1)) <= v < (1 << (bits - 1)):
        raise PaError(2, f"{what} = {v} does not fit a {bits}-bit signed integer")
    return v


def _int32_array(x, what):
    """A flat contiguous int32 copy of integer values x, refusing values a
    cast to int32 would wrap."""
    import numpy as np
    a = np.asarray(x)
    if a.size and a.dtype != np.int32:
        if not np.issubdtype(a.dtype, np.integer):
            raise PaError(3, f"{what} must be integers, got {a.dtype}")
        if int(a.min()) < -2**31 or int(a.max()) >= 2**31:
            raise PaError(2, f"{what} holds values outside int32")
    return np.ascontiguousarray(a, dtype=np.int32).reshape(-1)


class PaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "max_blocks_per_seq", "num_blocks", "partition_size")]


_lib = None


def library_path():
    return os.path.join(_HERE, LIB_NAME)


def load_library(path=None):
    """Load libpadecode.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  -- torch's HIP runtime must be loaded first
    p = path or library_path()
    if not os.path.exists(p):
        raise PaError(-1, f"{p} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    lib.pa_decode_workspace_bytes.argtypes = [ctypes.POINTER(PaShape)]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode.argtypes = [ctypes.POINTER(PaShape), vp, vp, vp, vp, vp, ctypes.c_float,
                              ctypes.c_int, ctypes.c_int, vp, vp, vp, ctypes.c_size_t, vp,
                              vp, vp]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [ctypes.POINTER(PaShape), vp, vp, vp, vp, vp, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_multi_workspace_bytes.argtypes = [ctypes.POINTER(PaShape), ctypes.c_int32]
    lib.pa_decode_multi_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_multi.argtypes = [ctypes.POINTER(PaShape), ctypes.c_int32, vp, vp, vp, vp, vp,
                                    ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                    ctypes.c_size_t, vp, vp, vp]
    lib.pa_decode_multi.restype = ctypes.c_int
    lib.pa_decode_prefix_workspace_bytes.argtypes = [ctypes.POINTER(PaShape)]
    lib.pa_decode_prefix_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode_prefix.argtypes = [ctypes.POINTER(PaShape), ctypes.c_int32, vp, vp, vp, vp, vp,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                     ctypes.c_size_t, vp, vp, vp]
    lib.pa_decode_prefix.restype = ctypes.c_int
    lib.pa_kv_append.argtypes = [ctypes.POINTER(PaShape), vp, vp, vp, vp, ctypes.c_int,
                                 ctypes.c_int, vp, vp, vp, vp, vp]
    lib.pa_kv_append.restype = ctypes.c_int
    lib.pa_lse_merge.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                 ctypes.c_int, vp, vp, vp]
    lib.pa_lse_merge.restype = ctypes.c_int
    lib.pa_workspace_reset.argtypes = [vp, ctypes.c_size_t, vp]
    lib.pa_workspace_reset.restype = ctypes.c_int
    lib.pa_status_str.argtypes = [ctypes.c_int]
    lib.pa_status_str.restype = ctypes.c_char_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.pa_pool_create.argtypes = [i32, ctypes.c_uint64, ctypes.POINTER(vp)]
    lib.pa_pool_create.restype = ctypes.c_int
    lib.pa_pool_destroy.argtypes = [vp]
    lib.pa_pool_destroy.restype = None
    lib.pa_pool_add_sequence.argtypes = [vp, i64, vp, i32, ctypes.POINTER(i32)]
    lib.pa_pool_add_sequence.restype = ctypes.c_int
    lib.pa_pool_append_token.argtypes = [vp, i64, i32]
    lib.pa_pool_append_token.restype = ctypes.c_int
    lib.pa_pool_free_sequence.argtypes = [vp, i64]
    lib.pa_pool_free_sequence.restype = ctypes.c_int
    lib.pa_pool_num_free.argtypes = [vp]
    lib.pa_pool_num_free.restype = i32
    lib.pa_pool_block_table.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.pa_pool_block_table.restype = ctypes.c_int
    lib.pa_pool_shared_prefix.argtypes = [vp, vp, i32, ctypes.POINTER(i32)]
    lib.pa_pool_shared_prefix.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_str(code):
    return load_library().pa_status_str(code).decode()


def _check(code):
    if code != 0:
        raise PaError(code, status_str(code))


def _torch_dtype_name(t):
    import torch
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
            torch.float8_e4m3fn: "fp8_e4m3", torch.uint8: "fp8_e4m3"}.get(t.dtype)


def make_shape(q, k_cache, block_table, partition_size):
    B, Hq, D = q.shape[0], q.shape[-2], q.shape[-1]
    dims = dict(batch=B, num_q_heads=Hq, num_kv_heads=k_cache.shape[1], head_dim=D,
                block_size=k_cache.shape[3], max_blocks_per_seq=block_table.shape[1],
                num_blocks=k_cache.shape[0], partition_size=partition_size)
    # the fields are int32: a wider value would wrap into one the library accepts
    return PaShape(**{k: _c_int(v, 32, k) for k, v in dims.items()})


def workspace_bytes(q, k_cache, block_table, partition_size):
    """Workspace bytes for a decode (q [B, Hq, D]) or multi-token (q [B, T, Hq, D]) call."""
    shape = make_shape(q, k_cache, block_table, partition_size)
    lib = load_library()
    if q.dim() == 4:
        return int(lib.pa_decode_multi_workspace_bytes(ctypes.byref(shape), q.shape[1]))
    return int(lib.pa_decode_workspace_bytes(ctypes.byref(shape)))


def prefix_workspace_bytes(q, k_cache, block_table):
    """Workspace bytes for a shared-prefix decode call (pa_decode_prefix)."""
    shape = make_shape(q, k_cache, block_table, SPLIT_BALANCED)
    return int(load_library().pa_decode_prefix_workspace_bytes(ctypes.byref(shape)))


def reset_workspace(workspace, stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    _check(load_library().pa_workspace_reset(workspace.data_ptr(), workspace.numel()
                                             * workspace.element_size(), s.cuda_stream))


def decode(q, k_cache, v_cache, block_table, context_lens, scale, *, k_scale=None,
           v_scale=None, partition_size=0, out=None, workspace=None, lse_out=None,
           stream=None, prefix_blocks=None):
    return prepare(q, k_cache, v_cache, block_table, context_lens, scale, k_scale=k_scale,
                   v_scale=v_scale, partition_size=partition_size, out=out,
                   workspace=workspace, lse_out=lse_out, stream=stream,
                   prefix_blocks=prefix_blocks)()


def decode_noalloc(q, k_cache, v_cache, block_table, context_lens, scale, *, k_scale=None,
                   v_scale=None, partition_size=0, out=None, lse_out=None, stream=None):
    """pa_decode_noalloc: as `decode` for q [B, Hq, D], with the split modes'
    partial results in the library's per-GPU scratch instead of a workspace
    (the C call allocates nothing; pass `out` to keep this call allocation-free
    on the Python side too). Calls that may overlap on one GPU race on that
    scratch. Returns out."""
    import torch
    lib = load_library()
    io = _torch_dtype_name(q)
    kv = _torch_dtype_name(k_cache)
    if io is None or kv is None or _torch_dtype_name(v_cache) != kv or q.dim() != 3:
        raise PaError(3, f"unsupported dtypes or rank: q={q.dtype} [{q.dim()}-d] k={k_cache.dtype}")
    if not q.is_cuda or not q.is_contiguous():
        raise PaError(2, "q must be a contiguous device tensor")
    if (k_cache.dim() != 5 or v_cache.dim() != 4 or block_table.dim() != 2
            or block_table.dtype != torch.int32 or context_lens.dtype != torch.int32):
        raise PaError(2, "expected k_cache [nb,Hkv,D/X,16,X], v_cache [nb,Hkv,D,16] and int32 "
                         "block_table [B,MBS], context_lens [B]")
    B, Hq, D = q.shape
    nb, Hkv = k_cache.shape[0], k_cache.shape[1]
    if (tuple(v_cache.shape) != (nb, Hkv, D, k_cache.shape[3])
            or k_cache.shape[2] * k_cache.shape[4] != D
            or tuple(block_table.shape[:1]) != (B,) or tuple(context_lens.shape) != (B,)):
        raise PaError(2, "inconsistent tensor shapes")
    check_buffers(q, (k_cache, v_cache, block_table, context_lens), out=out, lse_out=lse_out,
                  k_scale=k_scale, v_scale=v_scale, fp8=kv == "fp8_e4m3")
    if out is None:
        out = torch.empty_like(q)
    shape = make_shape(q, k_cache, block_table, partition_size)
    s = stream if stream is not None else torch.cuda.current_stream()
    _check(lib.pa_decode_noalloc(
        ctypes.byref(shape), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_table.data_ptr(), context_lens.data_ptr(), float(scale), DTYPE_CODE[io],
        DTYPE_CODE[kv], k_scale.data_ptr() if k_scale is not None else None,
        v_scale.data_ptr() if v_scale is not None else None, out.data_ptr(),
        lse_out.data_ptr() if lse_out is not None else None, s.cuda_stream))
    return out


class Prepared:
    """A pa_decode call with its arguments marshalled once; calling it enqueues
    the decode again on the same buffers (their contents may change)."""

    def __init__(self, fn, args, out, keep):
        self._fn = fn
        self._args = args
        self.out = out
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out


def _on_device(t):
    return t.is_cuda


def check_buffers(q, inputs, *, out=None, lse_out=None, workspace=None, k_scale=None,
                  v_scale=None, fp8=False, on_device=None):
    """Reject caller-supplied buffers the kernels would misuse, before anything
    is marshalled: every tensor on q's device and contiguous; out of q's dtype
    and shape; lse_out float32 of q's shape without the head dimension;
    k_scale / v_scale float32 [Hkv] (required for an fp8 cache); workspace a
    uint8 device tensor. Raises PaError(2) for a shape, layout or device
    mismatch and PaError(3) for a dtype mismatch. `on_device` decides what
    counts as device memory (tests pass their own to exercise the checks
    without a GPU)."""
    import torch
    dev_ok = on_device or _on_device
    Hkv = inputs[0].shape[1]

    def placed(name, t):
        if not dev_ok(t) or t.device != q.device:
            raise PaError(2, f"{name} must be on q's device ({q.device}), not {t.device}")
        if not t.is_contiguous():
            raise PaError(2, f"{name} must be contiguous")

    for name, t in zip(("k_cache", "v_cache", "block_table", "context_lens"), inputs):
        placed(name, t)
    if out is not None:
        placed("out", out)
        if out.dtype != q.dtype:
            raise PaError(3, f"out must have q's dtype {q.dtype}, not {out.dtype}")
        if tuple(out.shape) != tuple(q.shape):
            raise PaError(2, f"out must have q's shape {tuple(q.shape)}, not {tuple(out.shape)}")
    if lse_out is not None:
        placed("lse_out", lse_out)
        if lse_out.dtype != torch.float32:
            raise PaError(3, f"lse_out must be float32, not {lse_out.dtype}")
        if tuple(lse_out.shape) != tuple(q.shape[:-1]):
            raise PaError(2, "lse_out must have q's shape without the head dimension")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t is None:
            if fp8:
                raise PaError(1, f"{name} is required for an fp8 cache")
            continue
        placed(name, t)
        if t.dtype != torch.float32:
            raise PaError(3, f"{name} must be float32, not {t.dtype}")
        if tuple(t.shape) != (Hkv,):
            raise PaError(2, f"{name} must have shape [{Hkv}] (one per KV head)")
    if workspace is not None:
        placed("workspace", workspace)
        if workspace.dtype != torch.uint8:
            raise PaError(3, f"workspace must be a uint8 tensor, not {workspace.dtype}")


def prepare(q, k_cache, v_cache, block_table, context_lens, scale, *, k_scale=None,
            v_scale=None, partition_size=0, out=None, workspace=None, lse_out=None,
            stream=None, prefix_blocks=None):
    """out[b, h] = softmax(scale * q[b, h] . K^T) V over sequence b's paged cache.

    q [B, Hq, D] (float32 | float16 | bfloat16); k_cache [nb, Hkv, D/X, 16, X];
    v_cache [nb, Hkv, D, 16] (q's dtype, or float8_e4m3fn / uint8 codes with
    float32 k_scale, v_scale [Hkv]); block_table int32 [B, MBS];
    context_lens int32 [B]. partition_size: 0 = one pass per sequence, a
    positive multiple of 16 = split-K partitions of that many tokens,
    SPLIT_BALANCED = equal page shares per workgroup. `workspace` (uint8) is
    used when partition_size != 0; `workspace_bytes` gives its size. It must be
    zero-filled (reset_workspace) before first use and before a call whose
    counters take more bytes than the smallest counter bytes of any call since
    the last reset (a smaller call's partial results start right after its own
    counters, over a larger call's); every completed call leaves the counters
    it used zero, and a counter found stale makes that pair's rows NaN until
    the next reset (include/padecode.h). Without a workspace a zeroed one is
    allocated per call.

    q [B, T, Hq, D] selects the multi-token call (pa_decode_multi): T new
    tokens per sequence whose K/V are already in the cache, new token t seeing
    positions 0 .. L-T+t; out [B, T, Hq, D], lse_out [B, T, Hq].
    SPLIT_BALANCED works for any T there (equal pages per CU whatever the
    G * T rows per (sequence, KV head), G = Hq / Hkv).

    prefix_blocks (an int, q [B, Hq, D] and SPLIT_BALANCED only) selects the
    shared-prefix call (pa_decode_prefix): the rows' first prefix_blocks
    block-table entries are declared the same blocks (for a sequence, those
    among its full pages), and those pages are read once for all sequences; a
    row that breaks the declaration gets NaN outputs. Its workspace size is
    prefix_workspace_bytes.
    """
    import torch
    lib = load_library()
    if prefix_blocks is not None:
        prefix_blocks = _c_int(prefix_blocks, 32, "prefix_blocks")
    io = _torch_dtype_name(q)
    kv = _torch_dtype_name(k_cache)
    if io is None or kv is None or _torch_dtype_name(v_cache) != kv:
        raise PaError(3, f"unsupported dtypes q={q.dtype} k={k_cache.dtype} v={v_cache.dtype}")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("context_lens", context_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise PaError(2, f"{name} must be a contiguous device tensor")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise PaError(3, "block_table and context_lens must be int32")
    if q.dim() not in (3, 4) or k_cache.dim() != 5 or v_cache.dim() != 4 or block_table.dim() != 2:
        raise PaError(2, "expected q [B,Hq,D] or [B,T,Hq,D], k_cache [nb,Hkv,D/X,16,X], "
                         "v_cache [nb,Hkv,D,16]")
    multi = q.dim() == 4
    if prefix_blocks is not None and (multi or partition_size != SPLIT_BALANCED):
        raise PaError(2, "prefix_blocks needs q [B, Hq, D] and partition_size=SPLIT_BALANCED")
    B, Hq, D = q.shape[0], q.shape[-2], q.shape[-1]
    nb, Hkv = k_cache.shape[0], k_cache.shape[1]
    if (tuple(v_cache.shape) != (nb, Hkv, D, k_cache.shape[3])
            or k_cache.shape[2] * k_cache.shape[4] != D
            or tuple(block_table.shape[:1]) != (B,) or tuple(context_lens.shape) != (B,)):
        raise PaError(2, "inconsistent tensor shapes")
    check_buffers(q, (k_cache, v_cache, block_table, context_lens), out=out, lse_out=lse_out,
                  workspace=workspace, k_scale=k_scale, v_scale=v_scale, fp8=kv == "fp8_e4m3")
    if out is None:
        out = torch.empty_like(q)
    shape = make_shape(q, k_cache, block_table, partition_size)
    ws_ptr, ws_bytes = None, 0
    if partition_size:
        need = (prefix_workspace_bytes(q, k_cache, block_table) if prefix_blocks is not None
                else workspace_bytes(q, k_cache, block_table, partition_size))
        if workspace is None:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    ks = k_scale.data_ptr() if k_scale is not None else None
    vs = v_scale.data_ptr() if v_scale is not None else None
    s = stream if stream is not None else torch.cuda.current_stream()
    tail = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_table.data_ptr(), context_lens.data_ptr(), float(scale), DTYPE_CODE[io],
            DTYPE_CODE[kv], ks, vs, ws_ptr, ws_bytes, out.data_ptr(),
            lse_out.data_ptr() if lse_out is not None else None, s.cuda_stream)
    if multi:
        fn, args = lib.pa_decode_multi, (ctypes.byref(shape), q.shape[1]) + tail
    elif prefix_blocks is not None:
        fn, args = lib.pa_decode_prefix, (ctypes.byref(shape), prefix_blocks) + tail
    else:
        fn, args = lib.pa_decode, (ctypes.byref(shape),) + tail
    keep = (shape, q, k_cache, v_cache, block_table, context_lens, k_scale, v_scale,
            workspace, out, lse_out)
    return Prepared(fn, args, out, keep)


def kv_append(k_new, v_new, positions, block_table, k_cache, v_cache, *, k_scale=None,
              v_scale=None, stream=None):
    """Write k_new / v_new [B, Hkv, D] (float32 | float16 | bfloat16) into the
    caches at token positions[b] (int32 [B]; < 0 skips) through block_table,
    in place; an fp8 cache (float8_e4m3fn / uint8) quantises with the float32
    per-KV-head k_scale / v_scale. Returns (k_cache, v_cache)."""
    prepare_append(k_new, v_new, positions, block_table, k_cache, v_cache, k_scale=k_scale,
                   v_scale=v_scale, stream=stream)()
    return k_cache, v_cache


class PreparedAppend:
    """A pa_kv_append call with its arguments marshalled once."""

    def __init__(self, lib, args, keep):
        self._fn = lib.pa_kv_append
        self._args = args
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))


def prepare_append(k_new, v_new, positions, block_table, k_cache, v_cache, *, k_scale=None,
                   v_scale=None, stream=None):
    """Validate and marshal a kv_append call; calling the result enqueues it."""
    import torch
    lib = load_library()
    src = _torch_dtype_name(k_new)
    kv = _torch_dtype_name(k_cache)
    if (src not in ("f32", "f16", "bf16") or _torch_dtype_name(v_new) != src or kv is None
            or _torch_dtype_name(v_cache) != kv):
        raise PaError(3, f"unsupported dtypes k_new={k_new.dtype} k_cache={k_cache.dtype}")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("positions", positions),
                    ("block_table", block_table), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not t.is_cuda or not t.is_contiguous():
            raise PaError(2, f"{name} must be a contiguous device tensor")
    if positions.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise PaError(3, "positions and block_table must be int32")
    if k_new.dim() != 3 or tuple(v_new.shape) != tuple(k_new.shape) or k_cache.dim() != 5:
        raise PaError(2, "expected k_new, v_new [B,Hkv,D] and caches in the decode layout")
    B, H, D = k_new.shape
    nb = k_cache.shape[0]
    if (k_cache.shape[1] != H or k_cache.shape[2] * k_cache.shape[4] != D
            or tuple(v_cache.shape) != (nb, H, D, k_cache.shape[3])
            or tuple(positions.shape) != (B,) or block_table.dim() != 2
            or block_table.shape[0] != B):
        raise PaError(2, "inconsistent tensor shapes")
    fp8 = kv == "fp8_e4m3"
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t is None:
            if fp8:
                raise PaError(1, f"{name} is required for an fp8 cache")
            continue
        if not t.is_cuda or t.device != k_new.device or not t.is_contiguous():
            raise PaError(2, f"{name} must be a contiguous tensor on {k_new.device}")
        if t.dtype != torch.float32 or tuple(t.shape) != (H,):
            raise PaError(3, f"{name} must be float32 of shape [{H}]")
    for name, t in (("v_new", v_new), ("positions", positions), ("block_table", block_table),
                    ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.device != k_new.device:
            raise PaError(2, f"{name} must be on {k_new.device}, not {t.device}")
    shape = PaShape(batch=B, num_q_heads=H, num_kv_heads=H, head_dim=D,
                    block_size=k_cache.shape[3], max_blocks_per_seq=block_table.shape[1],
                    num_blocks=nb, partition_size=0)
    s = stream if stream is not None else torch.cuda.current_stream()
    args = (ctypes.byref(shape), k_new.data_ptr(), v_new.data_ptr(), positions.data_ptr(),
            block_table.data_ptr(), DTYPE_CODE[src], DTYPE_CODE[kv],
            k_scale.data_ptr() if k_scale is not None else None,
            v_scale.data_ptr() if v_scale is not None else None,
            k_cache.data_ptr(), v_cache.data_ptr(), s.cuda_stream)
    keep = (shape, k_new, v_new, positions, block_table, k_cache, v_cache, k_scale, v_scale)
    return PreparedAppend(lib, args, keep)


def lse_merge(shard_out, shard_lse, *, out=None, lse_out=None, stream=None):
    """Merge per-shard decode results: shard_out [S, ..., D] (float32 | float16 |
    bfloat16), shard_lse float32 [S, ...] (natural log) -> out [..., D] (and
    lse_out [...] if given). Returns out."""
    import torch
    lib = load_library()
    dt = _torch_dtype_name(shard_out)
    if dt not in ("f32", "f16", "bf16") or shard_lse.dtype != torch.float32:
        raise PaError(3, f"unsupported dtypes {shard_out.dtype}, {shard_lse.dtype}")
    for name, t in (("shard_out", shard_out), ("shard_lse", shard_lse)):
        if not t.is_cuda or not t.is_contiguous():
            raise PaError(2, f"{name} must be a contiguous device tensor")
    if shard_out.dim() < 2 or tuple(shard_lse.shape) != tuple(shard_out.shape[:-1]):
        raise PaError(2, "expected shard_out [S, ..., D] and shard_lse [S, ...]")
    S, D = shard_out.shape[0], shard_out.shape[-1]
    rows = shard_lse[0].numel()
    if shard_lse.device != shard_out.device:
        raise PaError(2, "shard_lse must be on shard_out's device")
    if out is None:
        out = torch.empty(shard_out.shape[1:], dtype=shard_out.dtype, device=shard_out.device)
    if (not out.is_cuda or out.device != shard_out.device or not out.is_contiguous()
            or out.dtype != shard_out.dtype or tuple(out.shape) != tuple(shard_out.shape[1:])):
        raise PaError(2, "out must be a contiguous tensor of shard_out's dtype, device and "
                         "shape without the shard dimension")
    if lse_out is not None and (not lse_out.is_cuda or lse_out.device != shard_out.device
                                or not lse_out.is_contiguous() or lse_out.dtype != torch.float32
                                or tuple(lse_out.shape) != tuple(shard_lse.shape[1:])):
        raise PaError(2, "lse_out must be a contiguous float32 tensor of shard_lse's shape "
                         "without the shard dimension, on shard_out's device")
    s = stream if stream is not None else torch.cuda.current_stream()
    _check(lib.pa_lse_merge(S, rows, D, shard_out.data_ptr(), shard_lse.data_ptr(),
                            DTYPE_CODE[dt], out.data_ptr(),
                            lse_out.data_ptr() if lse_out is not None else None, s.cuda_stream))
    return out


class BlockPool:
    """Host block pool with hash-chained prefix reuse (pa_pool_* in the C ABI):
    hands out the block ids of the tables `decode` and `kv_append` read.
    Token lists are int32; tables come back as numpy int32 arrays."""

    def __init__(self, num_blocks, seed=0):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check(self._lib.pa_pool_create(_c_int(num_blocks, 32, "num_blocks"), int(seed) & (2**64 - 1),
                                        ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_sequence(self, seq_id, tokens):
        """Register a sequence's prompt; returns the leading tokens found cached."""
        import numpy as np
        t = _int32_array(tokens, "tokens")
        got = ctypes.c_int32(0)
        _check(self._lib.pa_pool_add_sequence(self._h, _c_int(seq_id, 64, "seq_id"), t.ctypes.data,
                                              _c_int(t.size, 32, "the token count"),
                                              ctypes.byref(got)))
        return got.value

    def append_token(self, seq_id, token):
        _check(self._lib.pa_pool_append_token(self._h, _c_int(seq_id, 64, "seq_id"), _c_int(token, 32, "token")))

    def free_sequence(self, seq_id):
        _check(self._lib.pa_pool_free_sequence(self._h, _c_int(seq_id, 64, "seq_id")))

    def num_free(self):
        return self._lib.pa_pool_num_free(self._h)

    def shared_prefix(self, seq_ids):
        """Blocks the given sequences share from the start (prefix_blocks for
        a shared-prefix decode of exactly these sequences)."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        out = ctypes.c_int32(0)
        _check(self._lib.pa_pool_shared_prefix(self._h, ids.ctypes.data if ids.size else None, ids.size,
                                               ctypes.byref(out)))
        return int(out.value)

    def block_table(self, seq_ids, max_blocks, pad=0):
        """-> (int32 [len(seq_ids), max_blocks] block table, int32 context lengths)."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64).reshape(-1)
        mb = _c_int(max_blocks, 32, "max_blocks")
        if mb < 0:
            raise PaError(2, f"max_blocks = {mb} is negative")
        table = np.empty((ids.size, mb), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _check(self._lib.pa_pool_block_table(self._h, ids.ctypes.data, _c_int(ids.size, 32, "the sequence count"),
                                             mb, _c_int(pad, 32, "pad"), table.ctypes.data, lens.ctypes.data))
        return table, lens
