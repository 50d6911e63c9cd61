"""The five synthetic workloads of the CSA / HCA step, named by what they are.

Shapes follow the pages' statement of the method ([P1] "Token 的一生：DSV4 架构与
DSpark" §2.2: 256 raw tokens / 64 compressed entries per page, §3.2: top-512;
[P2] "DeepSeek-V4 的交錯壓縮注意力（CSA/HCA）" CSA / HCA paragraphs: 4x and ~128x
compression, sliding window). Only sizes, formats and seeds live here: no
arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field

KV_DIM = 576
TOPK = 512
RAW_PAGE = 256
C4_PAGE = 64
WINDOW = 128


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    seq_len: int | None            # raw length per sequence (None: ragged)
    kv_fmt: str                    # 'f32' or 'fp8' (FP8 e4m3 latent + bf16 RoPE)
    index_fmt: str                 # 'f32', 'fp8' or 'mxfp4'
    index_heads: int
    index_dim: int
    hadamard: bool
    heads: int                     # attention query heads
    q_dtype: str                   # 'f32' or 'bf16'
    out_dtype: str
    identity_pages: bool = False
    pool_pages: int | None = None  # physical pages in the pool (None: batch * pages/seq)
    new_tokens: int = 0            # prefill: new query tokens appended to the context
    hca_ratio: int = 0             # > 0: an HCA layer runs beside the CSA layer
    ragged: tuple = field(default=())  # (n_seqs, lo, hi) for log-uniform raw lengths
    q_len: int = 1                 # query tokens per sequence and step (multi-token decode)
    rope_dim: int = 0              # > 0: the step's indexer q / K rows get RoPE on their last rope_dim dims
    window: int = WINDOW
    softmax_scale: float = KV_DIM ** -0.5


TINY_FP32_DECODE = Workload(
    name="tiny_fp32_decode_L4096", seed=1001, batch=1, seq_len=4096, kv_fmt="f32",
    index_fmt="f32", index_heads=8, index_dim=64, hadamard=False, heads=16,
    q_dtype="f32", out_dtype="f32", identity_pages=True)

DECODE_128K = Workload(
    name="csa_decode_128k_b32", seed=1002, batch=32, seq_len=131072, kv_fmt="fp8",
    index_fmt="fp8", index_heads=64, index_dim=128, hadamard=True, heads=64,
    q_dtype="bf16", out_dtype="bf16", pool_pages=16384, rope_dim=64)

DECODE_1M = Workload(
    name="csa_decode_1m_b4", seed=1003, batch=4, seq_len=1048576, kv_fmt="fp8",
    index_fmt="mxfp4", index_heads=64, index_dim=128, hadamard=True, heads=128,
    q_dtype="bf16", out_dtype="bf16", pool_pages=16384, rope_dim=64)

SPEC_DECODE_128K = Workload(
    name="csa_spec_decode_128k_b32_q4", seed=1006, batch=32, seq_len=131072, kv_fmt="fp8",
    index_fmt="fp8", index_heads=64, index_dim=128, hadamard=True, heads=64,
    q_dtype="bf16", out_dtype="bf16", pool_pages=16384, q_len=4, rope_dim=64)

PREFILL_4K = Workload(
    name="csa_prefill_4096_on_128k", seed=1004, batch=1, seq_len=131072 + 4096, kv_fmt="fp8",
    index_fmt="fp8", index_heads=64, index_dim=128, hadamard=True, heads=64,
    q_dtype="bf16", out_dtype="bf16", new_tokens=4096, rope_dim=64)

HCA_RAGGED = Workload(
    name="hca_csa_ragged_b16", seed=1005, batch=16, seq_len=None, kv_fmt="fp8",
    index_fmt="fp8", index_heads=64, index_dim=128, hadamard=True, heads=64,
    q_dtype="bf16", out_dtype="bf16", hca_ratio=128, ragged=(16, 8192, 1048576), rope_dim=64)

ALL = (TINY_FP32_DECODE, DECODE_128K, DECODE_1M, SPEC_DECODE_128K, PREFILL_4K, HCA_RAGGED)
BY_NAME = {w.name: w for w in ALL}
