"""Plain CPU oracle of the compressed sparse attention (CSA) step and its heavily
compressed (HCA) mode.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library shares no
code with it, and nothing on the GPU path may call it.

Everything here is the plain definition written out in float64 with numpy:
no blocking, no fusion, no reordering. Where a floating-point value decides an
integer (a quantised code) the decision is taken in float32, the precision the
stored formats fix (fp32 scales, fp32 inputs to the rounding).

Sources (cited by page title and section):
  [P1] "Token 的一生：DSV4 架构与 DSpark" -- §1 (DSA -> DSV4 pipeline),
       §2.1 (C4 compressor: block [4k, 4k+3] emitted at position 4k+3),
       §2.2 (PagedIndexerMetadata: page_size 256, c4_page_size 64),
       §3.1 (FP8 / FP4 indexer query), §3.2 (top-512 transform), §4 (Hadamard).
  [P2] "DeepSeek-V4 的交錯壓縮注意力（CSA/HCA）：將百萬標記長上下文變為可用資源" --
       CSA paragraph (softmax-gated pooling with learned positional bias,
       light indexer, top-k compressed blocks, sliding-window branch),
       HCA paragraph (~128x compression, dense attention),
       "低精度與儲存策略的配合" (FP8 KV, BF16 RoPE dims, FP4 indexer).
  OCP 8-bit Floating Point Specification (OFP8) rev 1.0 for e4m3fn and the
  OCP Microscaling Formats (MX) v1.0 spec for MXFP4 (e2m1 + e8m0 per 32).

Readings where the pages are silent are listed in the repository's design
notes; each function states the one it takes.
"""
from __future__ import annotations

import numpy as np

KV_DIM = 576
LATENT_DIM = 512
ROPE_DIM = 64
TOPK = 512
RAW_PAGE = 256
C4_PAGE = 64

F32 = np.float32
FLT_MIN = float(np.finfo(np.float32).tiny)  # 2**-126

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------


def e4m3_value_table() -> np.ndarray:
    """Value of each of the 256 OCP e4m3fn codes (float64; NaN for 0x7F, 0xFF).

    OFP8 e4m3fn: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
    field 0 is subnormal (m/8 * 2**-6); S.1111.111 is NaN; no infinities.
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = e4m3_value_table()
E4M3_MAX = 448.0

# e2m1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; codes 0..7 are
# 0, 0.5, 1, 1.5, 2, 3, 4, 6 (MX v1.0, FP4 E2M1 element type).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0
E2M1_EMAX = 2  # exponent of the largest normal e2m1 value (4 = 2**2)


def _rne_to_grid(mag: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value to each non-negative magnitude, ties to
    the even index (the code whose mantissa LSB is 0). Magnitudes above the last
    grid value map to it (saturation). `grid` is ascending, grid[0] == 0."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.searchsorted(grid, mag, side="left")  # grid[hi-1] < mag <= grid[hi]
    hi = np.clip(hi, 1, len(grid) - 1)
    lo = hi - 1
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)
    return idx


_E4M3_POS = E4M3_VALUES[:127]  # codes 0x00..0x7E: 0 .. 448 ascending


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round to nearest e4m3fn code, ties to even, saturating at +-448.
    -0 encodes as 0x80 only if the input is -0.0 (sign is kept)."""
    v = np.asarray(v, dtype=np.float64)
    idx = _rne_to_grid(np.abs(v), _E4M3_POS).astype(np.uint8)
    return np.where(np.signbit(v), idx | np.uint8(0x80), idx).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern of x, rounding x (taken as float32) to nearest even."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Quantisers ([P1] §3.1, §4; [P2] "低精度與儲存策略的配合")
# ---------------------------------------------------------------------------


def quant_fp8_rows(v: np.ndarray):
    """Per-row FP8 quantisation of float32 rows (last axis = one token's vector).

    scale = max(amax, FLT_MIN) / 448 in float32, code = e4m3(fl32(v / scale)).
    Reading: one fp32 scale per row (per token / per head), OCP e4m3fn, RNE,
    saturating. Returns (codes uint8 [..., D], scale float32 [...]).
    """
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=-1)
    scale = (np.maximum(amax, F32(FLT_MIN)) / F32(E4M3_MAX)).astype(np.float32)
    ratio = (v / scale[..., None]).astype(np.float32)
    return e4m3_encode(ratio), scale


def dequant_fp8_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def quant_mxfp4_rows(v: np.ndarray):
    """MXFP4 quantisation (OCP MX v1.0) of float32 rows whose length is a
    multiple of 32: per block of 32, X = floor(log2(amax)) - emax(e2m1) with
    emax = 2 (X = -127 when the block is all zero), clamped to the e8m0 range
    [-127, 127]; code = e2m1(v / 2**X) rounded to nearest even, saturating at 6.

    Returns (packed uint8 [..., D/2] with element 2i in the low nibble,
             e8m0 scale bytes uint8 [..., D/32] = X + 127).
    """
    v = np.asarray(v, dtype=np.float32)
    D = v.shape[-1]
    assert D % 32 == 0
    blocks = v.reshape(v.shape[:-1] + (D // 32, 32)).astype(np.float64)
    amax = np.max(np.abs(blocks), axis=-1)
    _, e = np.frexp(amax)  # amax = m * 2**e, m in [0.5, 1) -> floor(log2 amax) = e - 1
    X = np.where(amax > 0, (e - 1) - E2M1_EMAX, -127)
    X = np.clip(X, -127, 127)
    scaled = blocks * np.exp2(-X.astype(np.float64))[..., None]  # exact: power of two
    mag_code = _rne_to_grid(np.abs(scaled), E2M1_VALUES).astype(np.uint8)
    code = np.where(np.signbit(scaled), mag_code | 8, mag_code)  # sign kept, as IEEE rounding does
    code = code.reshape(v.shape[:-1] + (D,)).astype(np.uint8)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def dequant_mxfp4_rows(packed: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    D = packed.shape[-1] * 2
    code = np.empty(packed.shape[:-1] + (D,), dtype=np.uint8)
    code[..., 0::2] = packed & 0xF
    code[..., 1::2] = packed >> 4
    mag = E2M1_VALUES[code & 7]
    val = np.where(code & 8, -mag, mag)
    X = np.asarray(scale_bytes, dtype=np.float64) - 127.0
    val = val.reshape(val.shape[:-1] + (D // 32, 32)) * np.exp2(X)[..., None]
    return val.reshape(val.shape[:-2] + (D,))


# ---------------------------------------------------------------------------
# Hadamard rotation ([P1] §4: rotate q and index-K before FP8/FP4 quantisation)
# ---------------------------------------------------------------------------


def hadamard_rotate(v: np.ndarray) -> np.ndarray:
    """y = H_D v / sqrt(D) along the last axis, H_D the Sylvester Hadamard matrix
    (H_1 = [1], H_2n = [[H, H], [H, -H]]), by the fast Walsh-Hadamard transform
    in float64. Reading: orthonormal scaling, natural (Sylvester) order."""
    y = np.array(v, dtype=np.float64, copy=True)
    D = y.shape[-1]
    assert D & (D - 1) == 0, "Hadamard size must be a power of two"
    h = 1
    while h < D:
        y = y.reshape(y.shape[:-1] + (D // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (D,))
        h *= 2
    return y / np.sqrt(D)


# ---------------------------------------------------------------------------
# Rotary position embedding of the indexer rows ([P1] §3.1: the indexer query
# is prepared by a fused rope -> hadamard -> quant step that takes a cos/sin
# table (`freqs_cis`) and the token positions; §4: the index-K rows go through
# the same rope -> hadamard -> quant before they are written to the cache)
# ---------------------------------------------------------------------------


def rope_cos_sin(pos, rope_dim: int, theta: float = 10000.0):
    """(cos, sin) float64 [len(pos), rope_dim/2] of the rotary angles
    pos * theta**(-2i/rope_dim), i = 0 .. rope_dim/2 - 1 (the textbook RoPE
    frequencies). Reading: the pages pass a precomputed table; this is what
    the table holds, before the caller stores it (float32) for the GPU."""
    pos = np.asarray(pos, dtype=np.float64).reshape(-1)
    i = np.arange(rope_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / rope_dim)
    ang = pos[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope_rotate(v: np.ndarray, cos: np.ndarray, sin: np.ndarray, rope_dim: int) -> np.ndarray:
    """Rotary embedding of the last rope_dim dims of each row, pairs (2i, 2i+1)
    of that slice rotated by the angle whose cosine and sine are cos[..., i],
    sin[..., i]:  x' = x cos - y sin,  y' = x sin + y cos  (float64).
    v [..., D]; cos, sin broadcast against [..., rope_dim/2]. Readings: the
    rotated dims are the last rope_dim of the row (the KV entry's layout puts
    its RoPE dims last), pairs are adjacent (the complex view of freqs_cis)."""
    y = np.array(v, dtype=np.float64, copy=True)
    D = y.shape[-1]
    r = y[..., D - rope_dim:]
    x0 = r[..., 0::2].copy()
    x1 = r[..., 1::2].copy()
    c = np.asarray(cos, dtype=np.float64)
    s_ = np.asarray(sin, dtype=np.float64)
    r[..., 0::2] = x0 * c - x1 * s_
    r[..., 1::2] = x0 * s_ + x1 * c
    return y


def index_prep(v: np.ndarray, hadamard: bool, fmt: str, rope=None):
    """Indexer row preparation ([P1] §3.1, §4): optional RoPE, optional
    Hadamard rotation, then quantisation to fmt ('fp8', 'mxfp4' or 'f32').
    The rotations are evaluated exactly in float64 and the result is rounded
    once to float32; the quantiser then takes its decisions on that float32
    value (the stored formats carry float32 scales).
    rope: None, or (cos, sin, rope_dim) with cos / sin broadcastable to
    [..., rope_dim/2] (the caller's table values for each row's position).
    Returns (codes, scale), or (float32 rows, None) for 'f32'."""
    x = np.asarray(v, dtype=np.float64)
    if rope is not None:
        cos, sin, rope_dim = rope
        x = rope_rotate(x, cos, sin, rope_dim)
    if hadamard:
        x = hadamard_rotate(x)
    x32 = x.astype(np.float32)
    if fmt == "fp8":
        return quant_fp8_rows(x32)
    if fmt == "mxfp4":
        return quant_mxfp4_rows(x32)
    if fmt == "f32":
        return x32, None
    raise ValueError(fmt)


def index_dequant(codes, scale, fmt: str) -> np.ndarray:
    if fmt == "fp8":
        return dequant_fp8_rows(codes, scale)
    if fmt == "mxfp4":
        return dequant_mxfp4_rows(codes, scale)
    return np.asarray(codes, dtype=np.float64)


# ---------------------------------------------------------------------------
# Compressor ([P1] §2.1; [P2] CSA and HCA paragraphs)
# ---------------------------------------------------------------------------


def compress_blocks(x: np.ndarray, start_pos: int, ratio: int, gate_w, gate_b) -> np.ndarray:
    """Softmax-gated pooling of complete blocks of `ratio` raw rows.

    Block k covers raw positions [ratio*k, ratio*k + ratio - 1] ([P1] §2.1 for
    ratio 4); rows of a partial tail block are not compressed. Per block:
        g_i = w . x_i + b[i]   (i = raw position mod ratio: learned positional bias)
        a   = softmax(g)
        c   = sum_i a_i x_i
    Reading: one scalar gate per raw token, output dim = input dim (576).
    x: [n, 576] rows at raw positions start_pos .. start_pos + n - 1.
    Returns float64 [n // ratio, 576].
    """
    assert start_pos % ratio == 0
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(gate_w, dtype=np.float64)
    b = np.asarray(gate_b, dtype=np.float64)
    nb = x.shape[0] // ratio
    out = np.empty((nb, x.shape[1]), dtype=np.float64)
    for k in range(nb):
        rows = x[k * ratio:(k + 1) * ratio]
        g = rows @ w + b[np.arange(ratio)]
        g = g - g.max()
        a = np.exp(g)
        a = a / a.sum()
        out[k] = a @ rows
    return out


def quant_kv_entries(c: np.ndarray, fmt: str):
    """Store KV entries ([P2] "低精度與儲存策略的配合": FP8 for most dims, BF16 for
    the RoPE dims). The entry is first taken to float32.
    fmt 'fp8': (latent e4m3 codes [n,512], scale f32 [n], rope bf16 bits [n,64]).
    fmt 'f32': (latent f32 [n,512], None, rope f32 [n,64])."""
    c32 = np.asarray(c, dtype=np.float64).astype(np.float32)
    if fmt == "fp8":
        codes, scale = quant_fp8_rows(c32[:, :LATENT_DIM])
        return codes, scale, bf16_bits(c32[:, LATENT_DIM:])
    if fmt == "f32":
        return c32[:, :LATENT_DIM].copy(), None, c32[:, LATENT_DIM:].copy()
    raise ValueError(fmt)


def dequant_kv_entries(latent, scale, rope, fmt: str) -> np.ndarray:
    """Exact float64 value of stored KV entries: [n, 576]."""
    if fmt == "fp8":
        lat = dequant_fp8_rows(latent, scale)
        rp = bf16_decode(rope)
    else:
        lat = np.asarray(latent, dtype=np.float64)
        rp = np.asarray(rope, dtype=np.float64)
    return np.concatenate([lat, rp], axis=-1)


# ---------------------------------------------------------------------------
# Paging ([P1] §2.2)
# ---------------------------------------------------------------------------


def page_slot(page_table_row: np.ndarray, j, page_size: int):
    """Physical slot of logical entry j: page_table[j // ps] * ps + j % ps."""
    j = np.asarray(j, dtype=np.int64)
    return np.asarray(page_table_row, dtype=np.int64)[j // page_size] * page_size + j % page_size


# ---------------------------------------------------------------------------
# Lightning indexer ([P1] §3; [P2] CSA paragraph)
# ---------------------------------------------------------------------------


def indexer_logits(q_hat: np.ndarray, w: np.ndarray, k_hat: np.ndarray) -> np.ndarray:
    """logits[j] = sum_h w[h] * max(0, q_hat[h] . k_hat[j]) for one query.
    q_hat [H_I, D], w [H_I], k_hat [n, D] (dequantised values). float64 [n]."""
    s = np.asarray(k_hat, dtype=np.float64) @ np.asarray(q_hat, dtype=np.float64).T
    return (np.maximum(s, 0.0) * np.asarray(w, dtype=np.float64)).sum(axis=1)


# ---------------------------------------------------------------------------
# Top-512 ([P1] §3.2)
# ---------------------------------------------------------------------------


def topk_logical(logits_row: np.ndarray, row_len: int, k: int = TOPK) -> np.ndarray:
    """Logical indices of the k largest logits among j < row_len, ranked by
    (logit descending, j ascending); -0 == +0 and NaN ranks last (numpy's sort
    order). Returned in ascending j order, length min(k, row_len)."""
    v = np.asarray(logits_row[:row_len], dtype=np.float64)
    j = np.arange(row_len)
    order = np.lexsort((j, -v))  # last key is primary
    return np.sort(order[:min(k, row_len)])


def topk_page_select(logits_row, row_len: int, page_table_row, c4_page_size: int = C4_PAGE,
                     k: int = TOPK):
    """(phys [k], logical [k]) int32 with -1 padding, ascending logical order."""
    sel = topk_logical(logits_row, row_len, k)
    logical = np.full(k, -1, dtype=np.int32)
    phys = np.full(k, -1, dtype=np.int32)
    logical[:len(sel)] = sel
    phys[:len(sel)] = page_slot(page_table_row, sel, c4_page_size)
    return phys, logical


# ---------------------------------------------------------------------------
# Attention ([P1] §1; [P2] CSA / HCA paragraphs)
# ---------------------------------------------------------------------------


def attend(q: np.ndarray, kv: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Multi-query attention of H query heads over E shared KV entries.
    score = scale * q . kv (576 dims); out = softmax(score) @ kv[:, :512].
    q [H, 576], kv [E, 576] -> float64 [H, 512]."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    s = softmax_scale * (q @ kv.T)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ kv[:, :LATENT_DIM]


def window_positions(p: int, window: int) -> np.ndarray:
    """Raw positions of the sliding window of a query at position p (inclusive)."""
    return np.arange(max(0, p - window + 1), p + 1)


def csa_attention_query(q, c4_kv_rows, raw_kv_rows, softmax_scale):
    """CSA for one query: one softmax over the selected compressed entries and
    the window's raw entries together (reading: no de-duplication)."""
    kv = np.concatenate([np.asarray(c4_kv_rows, np.float64).reshape(-1, KV_DIM),
                         np.asarray(raw_kv_rows, np.float64).reshape(-1, KV_DIM)], axis=0)
    return attend(q, kv, softmax_scale)


def hca_visible(p: int, ratio: int) -> int:
    """Number of HCA entries visible at position p: j with ratio*j + ratio-1 <= p."""
    return (p + 1) // ratio


def causal_row_len(p: int, n_entries: int, ratio: int = 4) -> int:
    """Visible compressed entries for a query at position p: 4j+3 <= p."""
    return min(n_entries, (p + 1) // ratio)


# ---------------------------------------------------------------------------
# One query of a decode / prefill step, composed from the definitions above
# ---------------------------------------------------------------------------


class KVPool:
    """Host copy of a KV pool in its stored form: latent [slots, 512] (e4m3
    codes or float32), scale [slots] (FP8 only), rope [slots, 64] (bf16 bits or
    float32); fmt 'fp8' or 'f32'."""

    def __init__(self, latent, scale, rope, fmt):
        self.latent, self.scale, self.rope, self.fmt = latent, scale, rope, fmt

    def rows(self, slots) -> np.ndarray:
        slots = np.asarray(slots, dtype=np.int64)
        sc = None if self.scale is None else self.scale[slots]
        return dequant_kv_entries(self.latent[slots], sc, self.rope[slots], self.fmt)


class IndexPool:
    """Host copy of an index-K pool: data [slots, ...], scale, fmt."""

    def __init__(self, data, scale, fmt):
        self.data, self.scale, self.fmt = data, scale, fmt

    def rows(self, slots) -> np.ndarray:
        slots = np.asarray(slots, dtype=np.int64)
        sc = None if self.scale is None else self.scale[slots]
        return index_dequant(self.data[slots], sc, self.fmt)


def csa_query(q_idx_hat, w, index_pool: IndexPool, c4_pool: KVPool, raw_pool: KVPool,
              page_table_row, raw_page_table_row, row_len: int, p: int, q_attn,
              window: int, softmax_scale: float, c4_page_size: int = C4_PAGE,
              raw_page_size: int = RAW_PAGE):
    """One query of the CSA step ([P1] §1 pipeline): score the row_len visible
    compressed entries, keep the top 512, attend over them and the window.
    Returns (logits float64 [row_len], selected logical j, out float64 [H, 512])."""
    slots = page_slot(page_table_row, np.arange(row_len), c4_page_size)
    logits = indexer_logits(q_idx_hat, w, index_pool.rows(slots))
    sel = topk_logical(logits, row_len)
    c4_rows = c4_pool.rows(page_slot(page_table_row, sel, c4_page_size))
    raw_rows = raw_pool.rows(page_slot(raw_page_table_row, window_positions(p, window), raw_page_size))
    return logits, sel, csa_attention_query(q_attn, c4_rows, raw_rows, softmax_scale)


def hca_query(hca_pool: KVPool, raw_pool: KVPool, hca_page_table_row, raw_page_table_row,
              p: int, ratio: int, q_attn, window: int, softmax_scale: float,
              hca_page_size: int = C4_PAGE, raw_page_size: int = RAW_PAGE):
    """One query of the HCA step ([P2] HCA paragraph): dense attention over every
    visible heavily compressed entry plus the window. float64 [H, 512]."""
    n = hca_visible(p, ratio)
    hca_rows = hca_pool.rows(page_slot(hca_page_table_row, np.arange(n), hca_page_size))
    raw_rows = raw_pool.rows(page_slot(raw_page_table_row, window_positions(p, window), raw_page_size))
    return csa_attention_query(q_attn, hca_rows, raw_rows, softmax_scale)


def dsa_query(q_idx_hat, w, index_pool: IndexPool, kv_pool: KVPool, page_table_row, p: int,
              q_attn, k: int, softmax_scale: float, page_size: int = 64):
    """One query of the DSA step, the ratio-1 mode ([P1] §1: in DSA the indexer
    scores the raw tokens, keeps the top-k and attention reads only their KV;
    §2.2: DSA pages hold 64 tokens). The query at raw position p sees tokens
    j <= p; there is no separate window (the recent tokens compete in the
    top-k like the rest). Returns (logits [p + 1], selected j, out [H, 512])."""
    n = p + 1
    slots = page_slot(page_table_row, np.arange(n), page_size)
    logits = indexer_logits(q_idx_hat, w, index_pool.rows(slots))
    sel = topk_logical(logits, n, k)
    rows = kv_pool.rows(page_slot(page_table_row, sel, page_size))
    return logits, sel, attend(q_attn, rows, softmax_scale)


# ---------------------------------------------------------------------------
# HiSparse staging ([P1] §5: the step's top-k compressed entries are swapped
# into a near tier for attention; entries selected again stay there)
# ---------------------------------------------------------------------------


class HotSet:
    """The near-tier state of one sequence: `hot_slots` slots, each empty (-1)
    or holding one logical entry, the reverse map, and each slot's last step
    of use."""

    def __init__(self, hot_slots: int):
        self.hot = hot_slots
        self.owner = [-1] * hot_slots
        self.slot_of = {}
        self.last_use = [0] * hot_slots


def hisparse_swap_in(state: HotSet, selected, step: int):
    """One step's staging of the selection `selected` (logical entries in
    order, -1 = empty). Entries already resident stay where they are. The
    others take, in selection order, the least recently used slots among those
    this step does not use -- empty slots first, then the oldest last use,
    equal stamps by the lower slot -- those slots taken in ascending order;
    a slot's previous entry leaves the near tier. Every slot used this step is
    stamped with `step`. Readings: least-recently-used replacement (the pages
    say only that hot entries stay near); the victims' order is ascending.
    Returns (near slot of each selected entry, -1 for -1; list of (entry, slot)
    copies made)."""
    hits = {j: state.slot_of[j] for j in selected if j >= 0 and j in state.slot_of}
    used = set(hits.values())
    misses = [j for j in selected if j >= 0 and j not in state.slot_of]
    free = [h for h in range(state.hot) if h not in used]
    free.sort(key=lambda h: (state.owner[h] >= 0, state.last_use[h] if state.owner[h] >= 0 else 0, h))
    victims = sorted(free[:len(misses)])
    assert len(victims) == len(misses), "more misses than free hot slots"
    copies = []
    for j, h in zip(misses, victims):
        old = state.owner[h]
        if old >= 0:
            del state.slot_of[old]
        state.owner[h] = j
        state.slot_of[j] = h
        copies.append((j, h))
    near = []
    for j in selected:
        if j >= 0:
            state.last_use[state.slot_of[j]] = step
            near.append(state.slot_of[j])
        else:
            near.append(-1)
    return near, copies
