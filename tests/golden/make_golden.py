"""Writes tests/golden/oracle_small_f16.json from the float64 oracle.

Calls only oracle/ (and the seeded input generator for the inputs). The file
freezes the oracle's output on one small case so that any later change to the
oracle's arithmetic shows up as a diff of this fixture.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from paged_kv_decode_05_amd import workloads as W  # noqa: E402

SPEC = W.Spec("golden_b2_h4kv2_d64_f16", 2, 4, 2, 64, "f16", "f16",
              ("fixed", [3, 21]), 2, ("fixed", 6), 0, 0, 2024)


def main():
    wl = W.make_workload(SPEC)
    out, lse = oracle.paged_decode_ref(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                       wl.context_lens, wl.scale, "f16", "f16",
                                       return_lse=True)
    doc = {
        "what": "float64 oracle output for the seeded spec below (regression fixture)",
        "spec": SPEC.__dict__ | {"lens": list(SPEC.lens[:1]) + [list(SPEC.lens[1])],
                                 "pool": list(SPEC.pool)},
        "out": [[[float.hex(float(v)) for v in row] for row in seq] for seq in out],
        "lse": [[float.hex(float(v)) for v in seq] for seq in lse],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_f16.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
