"""The decode calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed, on an MI355X: the split modes leave every counter they use at zero
when a call completes and clear nothing with a memset, so one capture can be
replayed any number of times on the same workspace. Each graph is replayed
several times with eager work and synchronisations in between and new query
values written into the captured buffer before each replay; every replay
must equal, bit for bit, an eager call on the same inputs."""
import numpy as np
import pytest
import torch

import paged_kv_decode_05_amd as pkd
from paged_kv_decode_05_amd import workloads as W

pytestmark = pytest.mark.gpu

BAL = pkd.SPLIT_BALANCED


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _replays(make_call, q, out, refill, n=3):
    """Capture make_call() (which writes `out`), then for each replay: new
    values into q, eager work, replay, and the eager call's result."""
    torch.cuda.synchronize()
    make_call()   # warm-up outside the capture (first-use lookups, lazy init)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        make_call()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    for i in range(n):
        refill(i)
        scratch.uniform_()                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        make_call()                        # the same call, eager
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(out)), f"replay {i}"
        assert torch.isfinite(got.float()).all(), f"replay {i}"


def _setup(spec, seed):
    wl = W.make_workload(spec, seed=seed)
    t = W.to_device(wl)
    rng = np.random.default_rng(seed)

    def refill(i):
        q = W._to_storage(W._normal(rng, wl.q.shape), spec.io_dtype)
        t["q"].copy_(W.storage_tensor(q, spec.io_dtype).to("cuda"))
    return wl, t, refill


@pytest.mark.parametrize("mode", ["partition512", "balanced"])
def test_decode_replays(mode):
    ps = 512 if mode == "partition512" else BAL
    spec = W.small_variant(W.SPECS[3], 8, ("uniform", 100, 3000))
    wl, t, refill = _setup(spec, 61)
    print(f"case graph decode {mode}", flush=True)
    out = torch.empty_like(t["q"])
    ws = torch.empty(pkd.workspace_bytes(t["q"], t["k_cache"], t["block_table"], ps), dtype=torch.uint8,
                     device="cuda")
    pkd.reset_workspace(ws)

    def call():
        pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                   float(wl.scale), partition_size=ps, out=out, workspace=ws)
    _replays(call, t["q"], out, refill)


def test_shared_prefix_replays():
    spec = W.small_variant(W.SPECS[5], 6, ("loguniform", 20, 30000))
    wl, t, refill = _setup(spec, 62)
    print("case graph shared prefix", flush=True)
    out = torch.empty_like(t["q"])
    ws = torch.empty(pkd.prefix_workspace_bytes(t["q"], t["k_cache"], t["block_table"]), dtype=torch.uint8,
                     device="cuda")
    pkd.reset_workspace(ws)

    def call():
        pkd.decode(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                   float(wl.scale), partition_size=BAL, out=out, workspace=ws,
                   prefix_blocks=spec.shared_prefix_tokens // 16)
    _replays(call, t["q"], out, refill)


def test_noalloc_replays():
    spec = W.small_variant(W.SPECS[3], 6, ("uniform", 100, 3000))
    wl, t, refill = _setup(spec, 63)
    print("case graph no-allocation balanced", flush=True)
    out = torch.empty_like(t["q"])

    def call():
        pkd.decode_noalloc(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
                           float(wl.scale), partition_size=BAL, out=out)
    _replays(call, t["q"], out, refill)


@pytest.mark.parametrize("ps", [0, BAL])
def test_multi_token_replays(ps):
    # eight new tokens per sequence: the wide-row kernels
    spec = W.small_variant(W.SPECS[3], 6, ("uniform", 100, 3000))
    wl, t, _ = _setup(spec, 64)
    rng = np.random.default_rng(65)
    q8 = W.storage_tensor(W.multi_query(wl, 8), spec.io_dtype).to("cuda")
    print(f"case graph multi-token T=8 ps={ps}", flush=True)
    out = torch.empty_like(q8)
    ws = None
    if ps:
        ws = torch.empty(pkd.workspace_bytes(q8, t["k_cache"], t["block_table"], ps), dtype=torch.uint8,
                         device="cuda")
        pkd.reset_workspace(ws)

    def refill(i):
        q = W._to_storage(W._normal(rng, tuple(q8.shape)), spec.io_dtype)
        q8.copy_(W.storage_tensor(q, spec.io_dtype).to("cuda"))

    def call():
        pkd.decode(q8, t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"], float(wl.scale),
                   partition_size=ps, out=out, workspace=ws)
    _replays(call, q8, out, refill)
