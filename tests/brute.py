"""Pure-Python brute force for paged decode attention on tiny inputs.

Written independently of oracle/: it decodes storage words with `struct`
(binary16 via the 'e' format, bfloat16 by widening to binary32) and fp8 via
torch's float8_e4m3fn type, and it locates every K/V element by explicit
flat-index arithmetic on the documented cache layout:

    K(blk, g, t, d) at ((((blk*Hkv + g)*(D//x) + d//x)*16 + t)*x + d%x)
    V(blk, g, t, d) at (((blk*Hkv + g)*D + d)*16 + t)

Scores, exponentials and sums are scalar Python floats (math.exp, math.fsum).
"""
import math
import struct

import numpy as np

BS = 16
EB = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}


def scalar_decoder(dtype):
    if dtype == "f32":
        return lambda w: float(w)
    if dtype == "f16":
        return lambda w: struct.unpack("<e", struct.pack("<H", int(w)))[0]
    if dtype == "bf16":
        return lambda w: struct.unpack("<f", struct.pack("<I", int(w) << 16))[0]
    if dtype == "fp8_e4m3":
        import torch
        table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn) \
            .to(torch.float64).tolist()
        return lambda w: table[int(w)]
    raise ValueError(dtype)


def brute_decode(q, k_cache, v_cache, block_table, context_lens, scale,
                 io_dtype, kv_dtype, k_scale=None, v_scale=None):
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    x = 16 // EB[kv_dtype]
    qd = scalar_decoder(io_dtype)
    kd = scalar_decoder(kv_dtype)
    kf = k_cache.reshape(-1)
    vf = v_cache.reshape(-1)
    qf = q.reshape(-1)
    sc = float(np.float32(scale))
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    lse = [[0.0] * Hq for _ in range(B)]
    for b in range(B):
        L = int(context_lens[b])
        for h in range(Hq):
            g = h // G
            ks = 1.0 if k_scale is None else float(np.float32(k_scale[g]))
            vs = 1.0 if v_scale is None else float(np.float32(v_scale[g]))
            qv = [qd(qf[(b * Hq + h) * D + d]) for d in range(D)]
            scores = []
            for t in range(L):
                blk = int(block_table[b][t // BS])
                slot = t % BS
                acc = []
                for d in range(D):
                    idx = ((((blk * Hkv + g) * (D // x) + d // x) * BS + slot) * x + d % x)
                    acc.append(qv[d] * kd(kf[idx]) * ks)
                scores.append(sc * math.fsum(acc))
            if L == 0:
                lse[b][h] = -math.inf
                continue
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            den = math.fsum(w)
            lse[b][h] = m + math.log(den)
            for d in range(D):
                terms = []
                for t in range(L):
                    blk = int(block_table[b][t // BS])
                    idx = (((blk * Hkv + g) * D + d) * BS + t % BS)
                    terms.append(w[t] * kd(vf[idx]) * vs)
                out[b][h][d] = math.fsum(terms) / den
    return np.array(out, dtype=np.float64), np.array(lse, dtype=np.float64)
