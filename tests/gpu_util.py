"""Helpers shared by the GPU tests."""
import numpy as np

from paged_kv_decode_05_amd.workloads import storage_tensor, to_device  # noqa: F401


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    e = np.abs(got - ref)
    return float(e.max()), float(e.mean())
