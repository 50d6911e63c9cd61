"""compressed_sparse_attention_c4_amd -- the CSA / HCA step of DeepSeek-V4 on
gfx950 (MI355X), behind the C ABI of include/csa.h.

This package is a thin ctypes binding: it takes torch tensors, passes their
device pointers, sizes and the current HIP stream to libcsa.so, and raises on
a non-OK status. Every step of the computation runs in the library's HIP
kernels; there is no fallback. Importing fails if libcsa.so is not built
(`python compressed_sparse_attention_c4_amd/build.py`).
"""
from __future__ import annotations

from ._binding import (  # noqa: F401
    CSA_OK, CSA_ERR_INVALID, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_HIP, CSA_ERR_BOUNDS,
    csa_set_debug, csa_debug_enabled,
    CSA_BF16, CSA_F32, CSA_FP8_E4M3, CSA_MXFP4, CSA_OP_CSA_ATTN, CSA_OP_HCA_ATTN,
    CSA_OP_INDEXER, CSA_OP_INDEXER_TOPK, CSA_OP_TOPK, CSA_OP_CSA_ATTN_F32, CSA_OP_HCA_ATTN_F32, CSA_PREP_HADAMARD, CSA_PREP_QUANT, CSA_PREP_ROPE,
    CSA_ROWS_PER_SEQ, CsaError,
    IndexPool, KvPool, LIB_PATH, c4_compress, csa_decode_prep, csa_index_prep, csa_sparse_attn,
    csa_status_string, csa_version, csa_workspace_size, hca_dense_attn, indexer_score,
    indexer_topk512, indexer_topk512_noalloc, lib, topk512_page_select, topk_page_select,
    CSA_OP_TOPK_K, CSA_TOPK_MAX, hisparse_swap_in,
    CSA_NOALLOC_SCRATCH_BYTES,
    CSA_TOPK, CSA_C4_PAGE, CSA_RAW_PAGE, CSA_C4_RATIO, CSA_HCA_RATIO,
)
from .pools import alloc_index_pool, alloc_kv_pool  # noqa: F401
