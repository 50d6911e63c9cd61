"""Helpers shared by the GPU parity tests: moving oracle-format pools (seeded
draws quantised by the oracle) to the library's device layout."""
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
