"""Fixtures under tests/golden/: E4M3 values worked by hand, and a frozen
oracle output (written by tests/golden/make_golden.py, which calls only the
oracle)."""
import json
import math
import os

import numpy as np

import oracle
from paged_kv_decode_05_amd import workloads as W

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_e4m3_spot_values_worked_by_hand():
    n = 0
    with open(os.path.join(HERE, "e4m3_spot_values.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            code, value = line.split()[:2]
            v = oracle.E4M3_TABLE[int(code, 16)]
            if value == "nan":
                assert math.isnan(v)
            else:
                assert v == float(value) and math.copysign(1, v) == math.copysign(1, float(value))
            n += 1
    assert n >= 15


def load_golden():
    with open(os.path.join(HERE, "oracle_small_f16.json")) as f:
        doc = json.load(f)
    s = doc["spec"]
    spec = W.Spec(s["name"], s["batch"], s["num_q_heads"], s["num_kv_heads"], s["head_dim"],
                  s["io_dtype"], s["kv_dtype"], (s["lens"][0], s["lens"][1]),
                  s["max_blocks_per_seq"], tuple(s["pool"]), s["partition_size"],
                  s["shared_prefix_tokens"], s["seed"])
    out = np.array([[[float.fromhex(v) for v in row] for row in seq] for seq in doc["out"]])
    lse = np.array([[float.fromhex(v) for v in seq] for seq in doc["lse"]])
    return spec, out, lse


def test_oracle_reproduces_frozen_fixture():
    spec, gout, glse = load_golden()
    wl = W.make_workload(spec)
    out, lse = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                       wl.context_lens, wl.scale, "f16", "f16",
                                       return_lse=True)
    np.testing.assert_allclose(out, gout, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, glse, rtol=0, atol=1e-14)
