"""Allocation of the paged pools the library reads and writes (torch device
memory; the library itself never allocates)."""
from __future__ import annotations

import torch

from ._binding import CSA_F32, CSA_FP8_E4M3, CSA_MXFP4, IndexPool, KvPool


def alloc_kv_pool(num_pages: int, page_size: int, fmt: int, device="cuda", poison=True) -> KvPool:
    """KV pool of num_pages pages. poison=True fills every byte with 0xFF
    (NaN in e4m3, bf16 and fp32) so that a read of an unwritten slot shows."""
    if fmt == CSA_FP8_E4M3:
        lat = torch.empty((num_pages, page_size, 512), dtype=torch.uint8, device=device)
        sc = torch.empty((num_pages, page_size), dtype=torch.float32, device=device)
        rope = torch.empty((num_pages, page_size, 64), dtype=torch.bfloat16, device=device)
    elif fmt == CSA_F32:
        lat = torch.empty((num_pages, page_size, 512), dtype=torch.float32, device=device)
        sc = None
        rope = torch.empty((num_pages, page_size, 64), dtype=torch.float32, device=device)
    else:
        raise ValueError(fmt)
    if poison:
        for t in (lat, sc, rope):
            if t is not None:
                t.view(torch.uint8).fill_(0xFF)
    return KvPool(lat, sc, rope, fmt, page_size)


def alloc_index_pool(num_pages: int, page_size: int, dim: int, fmt: int, device="cuda",
                     poison=True) -> IndexPool:
    if fmt == CSA_FP8_E4M3:
        data = torch.empty((num_pages, page_size, dim), dtype=torch.uint8, device=device)
        sc = torch.empty((num_pages, page_size), dtype=torch.float32, device=device)
    elif fmt == CSA_MXFP4:
        data = torch.empty((num_pages, page_size, dim // 2), dtype=torch.uint8, device=device)
        sc = torch.empty((num_pages, page_size, dim // 32), dtype=torch.uint8, device=device)
    elif fmt == CSA_F32:
        data = torch.empty((num_pages, page_size, dim), dtype=torch.float32, device=device)
        sc = None
    else:
        raise ValueError(fmt)
    if poison:
        for t in (data, sc):
            if t is not None:
                t.view(torch.uint8).fill_(0xFF)
    return IndexPool(data, sc, fmt, dim, page_size)
