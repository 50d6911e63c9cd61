"""Helpers shared by the GPU parity tests: moving oracle-format pools to the
device layout and back, and the near-rounding-midpoint exclusion used when a
quantisation decision may legitimately differ by one code between two correct
fp32 evaluations (different summation order in the rotation / pooling)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import csa_oracle as O

DEV = "cuda"


def t_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def kv_pool_to_device(pool: O.KVPool, page_size: int):
    import compressed_sparse_attention_c4_amd as csa
    n = pool.latent.shape[0]
    P = n // page_size
    if pool.fmt == "fp8":
        lat = t_dev(pool.latent.reshape(P, page_size, 512))
        sc = t_dev(pool.scale.reshape(P, page_size).astype(np.float32))
        rope = t_dev(pool.rope.reshape(P, page_size, 64).view(np.int16)).view(torch.bfloat16)
        return csa.KvPool(lat, sc, rope, csa.CSA_FP8_E4M3, page_size)
    lat = t_dev(pool.latent.reshape(P, page_size, 512).astype(np.float32))
    rope = t_dev(pool.rope.reshape(P, page_size, 64).astype(np.float32))
    return csa.KvPool(lat, None, rope, csa.CSA_F32, page_size)


def index_pool_to_device(pool: O.IndexPool, page_size: int, dim: int):
    import compressed_sparse_attention_c4_amd as csa
    n = pool.data.shape[0]
    P = n // page_size
    if pool.fmt == "fp8":
        return csa.IndexPool(t_dev(pool.data.reshape(P, page_size, dim)),
                             t_dev(pool.scale.reshape(P, page_size).astype(np.float32)),
                             csa.CSA_FP8_E4M3, dim, page_size)
    if pool.fmt == "mxfp4":
        return csa.IndexPool(t_dev(pool.data.reshape(P, page_size, dim // 2)),
                             t_dev(pool.scale.reshape(P, page_size, dim // 32)),
                             csa.CSA_MXFP4, dim, page_size)
    return csa.IndexPool(t_dev(pool.data.reshape(P, page_size, dim).astype(np.float32)), None,
                         csa.CSA_F32, dim, page_size)


def fp8_codes_match(gpu_codes, ora_codes, ora_ratio, rel=1e-5):
    """GPU and oracle e4m3 codes decode to the same value (+0 and -0 are the
    same value), except adjacent codes where the oracle's pre-rounding value
    (ora_ratio = v / scale in fp32, in code units up to 448) lies within
    rel * (|midpoint| + 16) of the midpoint between them: the rounding error of
    an fp32 sum is on the scale of its inputs, not of each output element.
    Returns (ok, n_mismatch)."""
    g = np.asarray(gpu_codes).astype(np.int64).ravel()
    o = np.asarray(ora_codes).astype(np.int64).ravel()
    r = np.asarray(ora_ratio, dtype=np.float64).ravel()
    bad = np.flatnonzero(O.E4M3_VALUES[g] != O.E4M3_VALUES[o])
    for i in bad:
        a, b = O.E4M3_VALUES[g[i]], O.E4M3_VALUES[o[i]]
        mid = (a + b) / 2
        if abs(r[i] - mid) > rel * (abs(mid) + 16.0):
            return False, len(bad)
        # adjacent on the number line: no representable value strictly between
        lo, hi = min(a, b), max(a, b)
        fin = O.E4M3_VALUES[np.isfinite(O.E4M3_VALUES)]
        if np.any((fin > lo) & (fin < hi)):
            return False, len(bad)
    return True, len(bad)


def unpack_e2m1(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
