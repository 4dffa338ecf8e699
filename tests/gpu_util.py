"""Helpers shared by GPU tests, smoke() and bench.py: upload a seeded
workload to device tensors and compare against the oracle."""
import numpy as np
import torch

TORCH_IO = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def storage_tensor(raw, dtype):
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == "f32":
        return t
    if dtype in ("f16", "bf16"):
        return t.view(torch.int16).view(TORCH_IO[dtype])
    if dtype == "fp8_e4m3":
        return t.view(torch.uint8)
    raise ValueError(dtype)


def to_device(wl, device="cuda:0"):
    s = wl.spec
    d = {
        "q": storage_tensor(wl.q, s.io_dtype).to(device),
        "k_cache": storage_tensor(wl.k_cache, s.kv_dtype).to(device),
        "v_cache": storage_tensor(wl.v_cache, s.kv_dtype).to(device),
        "block_table": torch.from_numpy(wl.block_table).to(device),
        "context_lens": torch.from_numpy(wl.context_lens).to(device),
        "k_scale": None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(device),
        "v_scale": None if wl.v_scale is None else torch.from_numpy(wl.v_scale).to(device),
    }
    return d


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    e = np.abs(got - ref)
    return float(e.max()), float(e.mean())
