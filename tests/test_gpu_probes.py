"""GPU probes of the building blocks the kernels assume (test-only library
tests/probes/libpaprobes.so): MFMA operand/accumulator lane layouts and exact
E4M3 widening. Inputs are small and in bounds."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
PROBES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libpaprobes.so")


def lib():
    import paged_kv_decode_05_amd as pkd
    pkd.load_library()              # torch first, then one HIP runtime for both
    L = ctypes.CDLL(PROBES)
    L.pa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p]
    L.pa_probe_fp8.argtypes = [ctypes.c_void_p] * 4
    L.pa_probe_permlane.argtypes = [ctypes.c_void_p] * 3
    return L


@pytest.mark.parametrize("which,k,dt", [(0, 32, torch.float16), (1, 32, torch.bfloat16),
                                        (2, 16, torch.float16), (3, 16, torch.bfloat16),
                                        (4, 4, torch.float32)])
def test_mfma_lane_layout(which, k, dt):
    print(f"probe mfma which={which}", flush=True)
    g = torch.Generator().manual_seed(which)
    A = torch.randint(-8, 9, (16, k), generator=g).to(dt)
    B = torch.randint(-8, 9, (k, 16), generator=g).to(dt)
    C = torch.zeros(16, 16, dtype=torch.float32, device="cuda")
    Ad, Bd = A.cuda().contiguous(), B.cuda().contiguous()
    s = torch.cuda.current_stream()
    assert lib().pa_probe_mfma(which, Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(),
                               s.cuda_stream) == 0
    torch.cuda.synchronize()
    ref = A.double() @ B.double()
    assert torch.equal(C.cpu().double(), ref)


def test_fp8_widening_is_exact():
    print("probe fp8", flush=True)
    codes = torch.arange(256, dtype=torch.uint8).cuda()
    o16 = torch.zeros(256, dtype=torch.int16, device="cuda")
    ob = torch.zeros(256, dtype=torch.int16, device="cuda")
    s = torch.cuda.current_stream()
    assert lib().pa_probe_fp8(codes.data_ptr(), o16.data_ptr(), ob.data_ptr(),
                              s.cuda_stream) == 0
    torch.cuda.synchronize()
    f16 = o16.cpu().view(torch.float16).double().numpy()
    bf = ob.cpu().view(torch.bfloat16).double().numpy()
    ref = oracle.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(f16), nan) and np.array_equal(np.isnan(bf), nan)
    assert np.array_equal(f16[~nan], ref[~nan])
    assert np.array_equal(bf[~nan], ref[~nan])


def test_permlane_swaps_pair_lanes_16_and_32_apart():
    # with the same register in both operands, the 16-lane swap must hand
    # lane l the values of lanes l and l^16, the 32-lane swap those of l and
    # l^32 (the head reductions take max / sum of the pair)
    print("probe permlane", flush=True)
    vals = torch.arange(1000, 1064, dtype=torch.int32).cuda()
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    assert lib().pa_probe_permlane(vals.data_ptr(), out.data_ptr(), s.cuda_stream) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(64, 4)
    for l in range(64):
        assert sorted(o[l, :2]) == sorted([1000 + l, 1000 + (l ^ 16)]), (l, o[l])
        assert sorted(o[l, 2:]) == sorted([1000 + l, 1000 + (l ^ 32)]), (l, o[l])
