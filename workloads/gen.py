"""Seeded synthetic input draws shared by the tests, the smoke check and the
benchmark. Only random draws, permutations and storage-type casts live here:
none of the method's arithmetic (no compression, rotation, quantisation,
scoring, selection or attention).

Host draws use numpy's PCG64 (`numpy.random.default_rng(seed)`); large device
draws use torch's Philox generator on the GPU with the same seed. Value
distributions: KV and q values N(0, 1), indexer head weights U(0, 1), gate
weights N(0, 1/576), positional gate biases N(0, 0.1) (variance 0.1).
"""
from __future__ import annotations

import math

import numpy as np

KV_DIM = 576


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    return (g.standard_normal(shape) * std).astype(np.float32)


def uniform(g: np.random.Generator, shape, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    return g.uniform(lo, hi, shape).astype(np.float32)


def gate_params(g: np.random.Generator, ratio: int):
    """(w [576] ~ N(0, 1/576), b [ratio] ~ N(0, 0.1)) as float32."""
    w = normal(g, (KV_DIM,), std=1.0 / math.sqrt(KV_DIM))
    b = normal(g, (ratio,), std=math.sqrt(0.1))
    return w, b


def page_table(g: np.random.Generator, batch: int, pages_per_seq: int, num_pages: int,
               identity: bool = False) -> np.ndarray:
    """int32 [batch, pages_per_seq]: distinct physical page ids, a random
    permutation of range(num_pages) (or the identity)."""
    need = batch * pages_per_seq
    assert need <= num_pages
    ids = np.arange(num_pages, dtype=np.int32) if identity else g.permutation(num_pages).astype(np.int32)
    return ids[:need].reshape(batch, pages_per_seq).copy()


def ragged_lengths(g: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n raw lengths floor(exp(U(ln lo, ln hi))), int64."""
    return np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), n))).astype(np.int64)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Storage cast of a float32 draw to bfloat16 (torch's CPU cast), as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def device_normal(shape, seed: int, device="cuda", dtype=None, std: float = 1.0):
    """Large N(0, std) draw made on the device with a seeded torch generator."""
    import torch
    dtype = dtype or torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def device_uniform(shape, seed: int, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.rand(shape, generator=gen, device=device, dtype=torch.float32)


def rope_rows(positions, rope_dim: int, theta: float = 10000.0) -> np.ndarray:
    """Rows of the rotary-embedding table at the given positions, float32
    [len(positions), rope_dim/2, 2]: (cos, sin) of the angle p * theta^(-2i/rope_dim)
    of pair i at position p, evaluated in float64, stored as float32."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / rope_dim)
    ang = np.asarray(positions, dtype=np.float64).reshape(-1)[:, None] * inv[None, :]
    out = np.empty(ang.shape + (2,), dtype=np.float32)
    out[..., 0] = np.cos(ang)
    out[..., 1] = np.sin(ang)
    return out


def rope_table(max_pos: int, rope_dim: int, theta: float = 10000.0) -> np.ndarray:
    """The caller's rotary-embedding table, float32 [max_pos, rope_dim/2, 2],
    rows 0 .. max_pos - 1 of rope_rows (the textbook RoPE table; an input of
    the indexer preparation, like the head weights)."""
    out = np.empty((max_pos, rope_dim // 2, 2), dtype=np.float32)
    step = 1 << 16
    for p0 in range(0, max_pos, step):
        out[p0:p0 + step] = rope_rows(np.arange(p0, min(max_pos, p0 + step)), rope_dim, theta)
    return out
