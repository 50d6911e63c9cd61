"""Oracle side of the full-size checks.

A device workload (workloads.device) fills its pools through the library from
seeded raw draws and then runs one step. Here the oracle rebuilds, for a few
sampled sequences or query rows, what the pools hold after that step: the
same raw draws are taken again from the seeded generator (workloads.gen, the
only code both sides share) and everything else -- rotation, quantisation,
compression, scoring, selection, attention -- is the oracle's own. Nothing
the library wrote is read back as an oracle input.

Each rebuild is held in logical order (entry j of the sequence at row j), so
the oracle's query functions run with an identity page table.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import csa_oracle as O
from tests import quant_band as Q
from workloads import gen
from workloads.device import _CHUNK


def regen_fill_rows(slots, dim: int, seed: int, total_slots: int) -> np.ndarray:
    """Raw draws of the pool fills (device.fill_index_pool /
    fill_kv_pool_physical): physical row r comes from chunk r // 2^17 of
    device_normal((n, dim), seed * 1000 + chunk). float32 [len(slots), dim]."""
    slots = np.asarray(slots, dtype=np.int64)
    out = np.empty((len(slots), dim), np.float32)
    chunks = slots // _CHUNK
    for c in np.unique(chunks):
        sel = np.flatnonzero(chunks == c)
        n = min(_CHUNK, total_slots - int(c) * _CHUNK)
        v = gen.device_normal((n, dim), seed * 1000 + int(c))
        idx = torch.as_tensor(slots[sel] - int(c) * _CHUNK, device=v.device)
        out[sel] = v[idx].float().cpu().numpy()
        del v
    return out


def rope_cs(positions, rope_dim):
    """(cos, sin) float64 [len(positions), rope_dim/2] of the RoPE table the
    library was given (the float32 values of the seeded input table)."""
    cs = gen.rope_rows(positions, rope_dim).astype(np.float64)
    return cs[..., 0], cs[..., 1]


def host(t: torch.Tensor) -> np.ndarray:
    """A seeded device draw (an input, not a library result) as float32."""
    return t.float().cpu().numpy()


def identity_pages(n_entries: int, page: int) -> np.ndarray:
    return np.arange((n_entries + page - 1) // page, dtype=np.int64)


class LazyKVPool:
    """Oracle KV pool in logical order whose rows are produced on demand:
    rows(j) quantises and dequantises the raw entries kv_fn(j) (per-entry
    quantisation, so a subset quantises exactly as the whole would)."""

    def __init__(self, kv_fn, fmt: str):
        self.kv_fn, self.fmt = kv_fn, fmt

    def rows(self, j) -> np.ndarray:
        j = np.asarray(j, dtype=np.int64)
        lat, sc, rope = O.quant_kv_entries(self.kv_fn(j), self.fmt)
        return O.dequant_kv_entries(lat, sc, rope, self.fmt)


class SeqState:
    """Oracle copy of one sequence's index-K rows, compressed KV entries and
    raw window rows after the step, with the query inputs of one row.

    Besides the oracle's own quantised rows it keeps, for every index-K row
    and query element, the value step a correct float32 evaluation of the
    rotation may legitimately take instead (tests/quant_band.py): nonzero only
    where the exact value lies within the evaluation band of a rounding
    midpoint. The logit tolerance of an entry is widened by exactly what those
    steps can change."""

    def __init__(self, wl, kraw, kv_fn, raw_pos0, raw_rows, q_idx, w_idx, q_attn, p, row_len,
                 bands: bool = True, k_rope=None):
        """k_rope: None, or (rows, positions): the index-K rows written by the
        step, which the library rotated (RoPE) at those positions."""
        self.wl = wl
        kin = np.asarray(kraw, dtype=np.float64)
        if k_rope is not None and wl.rope_dim:
            rows, kpos = k_rope
            kin = kin.copy()
            cos, sin = rope_cs(kpos, wl.rope_dim)
            kin[rows] = O.rope_rotate(kin[rows], cos, sin, wl.rope_dim)  # exact; then index_prep rounds once
        codes, sc = O.index_prep(kin, wl.hadamard, wl.index_fmt)
        self.ipool = O.IndexPool(codes, sc, wl.index_fmt)
        self.dk = None
        if bands:
            self.dk = Q.band_delta(Q.exact_rotated(kin, wl.hadamard),
                                   Q.rotation_error_bound(kraw, wl.index_dim, rope=bool(wl.rope_dim)),
                                   wl.index_fmt)
        self.c4 = LazyKVPool(kv_fn, wl.kv_fmt)
        self.raw = O.KVPool(*O.quant_kv_entries(raw_rows, wl.kv_fmt), wl.kv_fmt)
        self._raw_rows = raw_rows
        self.raw_pos0 = raw_pos0
        self.q_idx, self.w_idx, self.q_attn = q_idx, w_idx, q_attn
        self.p, self.row_len = p, row_len
        self.q_pos = p  # the query's RoPE position
        self.n_entries = kraw.shape[0]

    def raw_map(self) -> np.ndarray:
        """'page table' with page size 1 sending raw position -> row here."""
        m = np.zeros(self.p + 1, dtype=np.int64)
        m[self.raw_pos0:] = np.arange(self.p + 1 - self.raw_pos0)
        return m

    def q_rope(self):
        """The oracle's RoPE argument for the query rows (None without RoPE)."""
        if not self.wl.rope_dim:
            return None
        cos, sin = rope_cs([self.q_pos], self.wl.rope_dim)
        return cos, sin, self.wl.rope_dim

    def scores(self):
        """(oracle logits [row_len], slack [row_len]): the slack bounds what
        in-band codes of the query and of each index-K row can change."""
        wl = self.wl
        qc, qs = O.index_prep(self.q_idx, wl.hadamard, wl.index_fmt, rope=self.q_rope())
        qhat = O.index_dequant(qc, qs, wl.index_fmt)
        n = self.row_len
        khat = self.ipool.rows(np.arange(n))
        logits = O.indexer_logits(qhat, self.w_idx, khat)
        dq = Q.band_delta(Q.exact_rotated(self.q_idx, wl.hadamard, rope=self.q_rope()),
                          Q.rotation_error_bound(self.q_idx, wl.index_dim, rope=bool(wl.rope_dim)),
                          wl.index_fmt)
        return logits, Q.logit_slack(qhat, dq, self.w_idx, khat, self.dk[:n])

    def oracle_query(self):
        """The oracle's whole step for this query row ([P1] §1 pipeline): query
        preparation, logits of every visible entry, top-512, attention over the
        selection and the window. (logits, selected j, out [H, 512])."""
        wl = self.wl
        qc, qs = O.index_prep(self.q_idx, wl.hadamard, wl.index_fmt, rope=self.q_rope())
        qhat = O.index_dequant(qc, qs, wl.index_fmt)
        return O.csa_query(qhat, self.w_idx, self.ipool, self.c4, self.raw,
                           identity_pages(self.n_entries, 64), self.raw_map(), self.row_len, self.p,
                           self.q_attn, wl.window, wl.softmax_scale, c4_page_size=64,
                           raw_page_size=1)

    def attend(self, sel) -> np.ndarray:
        """Oracle attention [H, 512] over the compressed entries `sel` (logical
        indices) and the query's window."""
        wl = self.wl
        c4_rows = self.c4.rows(np.asarray(sel, dtype=np.int64))
        win = self.raw_map()[O.window_positions(self.p, wl.window)]
        return O.csa_attention_query(self.q_attn, c4_rows, self.raw.rows(win), wl.softmax_scale)


def decode_raw_tail(W, b: int, stepped: bool):
    """(first position, rows) of sequence b's raw rows in the window pool: the
    tail draw (positions L - n .. L - 1), and after a step the current token
    stored over position L - 1."""
    L = int(W.lens[b])
    tails = np.minimum(W.lens, 2 * 256)
    cu = np.concatenate([[0], np.cumsum(tails)])
    x_tail = host(gen.device_normal((int(cu[-1]), 576), W.seed + 3))[cu[b]:cu[b + 1]]
    raw_pos0 = L - int(tails[b])
    rows = x_tail.astype(np.float64)
    if stepped and W.with_compress:
        x_tok = host(W.x_new).reshape(W.B, 4, 576)[b, 3:4]
        rows[L - 1 - raw_pos0] = O.compress_blocks(x_tok, L - 1, 1, np.zeros(576), np.zeros(1))[0]
    return raw_pos0, rows


def decode_seq(W, b: int, bands: bool = True) -> SeqState:
    """Sequence b of a CsaDecode after one step."""
    wl = W.wl
    L, N = int(W.lens[b]), int(W.N[b])
    total = W.P * 64
    pt = W.pt_host[b]
    kraw = regen_fill_rows(O.page_slot(pt, np.arange(N), 64), wl.index_dim, W.seed + 1, total)
    last = None
    if W.with_compress and L % 4 == 0:  # the current token completes block N-1
        x_new = host(W.x_new).reshape(W.B, 4, 576)[b]
        last = O.compress_blocks(x_new, L - 4, 4, host(W.gate_w), host(W.gate_b))[0]
        kraw[N - 1] = host(W.k_new)[b]

    def kv_fn(j):
        rows = regen_fill_rows(O.page_slot(pt, j, 64), 576, W.seed + 2, total).astype(np.float64)
        if last is not None:
            rows[j == N - 1] = last
        return rows

    raw_pos0, raw_rows = decode_raw_tail(W, b, stepped=True)
    k_rope = ([N - 1], [L - 1]) if last is not None else None
    return SeqState(wl, kraw, kv_fn, raw_pos0, raw_rows, host(W.q_idx)[b], host(W.w_idx)[b],
                    host(W.q_attn)[b], L - 1, N, bands=bands, k_rope=k_rope)


def spec_decode_row(W, t: int, bands: bool = True) -> SeqState:
    """Query row t of a CsaSpecDecode after one step: sequence b = t // 4 at
    position L - 4 + t % 4; the step stored the block's four rows at raw
    positions L - 4 .. L - 1 and completed block N - 1."""
    b = t // W.wl.q_len
    st = decode_seq(W, b, bands=bands)
    L = int(W.lens[b])
    x_new = host(W.x_new).reshape(W.B, 4, 576)[b]
    for i in range(3):
        st_row = O.compress_blocks(x_new[i:i + 1], L - 4 + i, 1, np.zeros(576), np.zeros(1))[0]
        rows = np.array(st._raw_rows)
        rows[L - 4 + i - st.raw_pos0] = st_row
        st._raw_rows = rows
    st.raw = O.KVPool(*O.quant_kv_entries(st._raw_rows, W.wl.kv_fmt), W.wl.kv_fmt)
    st.q_idx, st.w_idx, st.q_attn = host(W.q_idx)[t], host(W.w_idx)[t], host(W.q_attn)[t]
    st.p, st.row_len = int(W.pos_host[t]), int(W.rows_len_host[t])
    st.q_pos = st.p
    return st


def hca_oracle(Wh, b: int) -> np.ndarray:
    """HCA output of sequence b of an HcaCsaRagged step: every visible HCA
    entry plus the window, which the HCA layer reads before the CSA layer
    stores the current token. float64 [H, 512]."""
    return hca_query_of(*hca_state(Wh, b))


def hca_query_of(pool, raw, m, L, q, wl) -> np.ndarray:
    n = L // wl.hca_ratio
    return O.hca_query(pool, raw, identity_pages(max(n, 1), 64), m, L - 1, wl.hca_ratio,
                       q, wl.window, wl.softmax_scale, hca_page_size=64, raw_page_size=1)


def hca_state(Wh, b: int):
    """The oracle's inputs of sequence b's HCA query: (HCA pool in logical
    order, raw window pool, raw position map, L, query, workload)."""
    wl = Wh.wl
    L = int(Wh.lens[b])
    n = L // wl.hca_ratio
    slots = O.page_slot(Wh.hpt_host[b], np.arange(n), 64)
    rows = regen_fill_rows(slots, 576, Wh.hca_seed, Wh.Ph * 64)
    pool = O.KVPool(*O.quant_kv_entries(rows, wl.kv_fmt), wl.kv_fmt)
    raw_pos0, raw_rows = decode_raw_tail(Wh.csa, b, stepped=False)
    raw = O.KVPool(*O.quant_kv_entries(raw_rows, wl.kv_fmt), wl.kv_fmt)
    m = np.zeros(L, dtype=np.int64)
    m[raw_pos0:] = np.arange(L - raw_pos0)
    return pool, raw, m, L, host(Wh.q_hca)[b], wl


def prefill_row(W, t: int, bands: bool = True) -> SeqState:
    """Query row t (position ctx + t) of a CsaPrefill after its step."""
    wl = W.wl
    ctx, new = W.ctx, W.new
    pos = ctx + t
    n_vis = int(W.row_len_host[t])
    total = W.P * 64
    pt = W.pt_host[0]
    e0 = ctx // 4
    kraw = regen_fill_rows(O.page_slot(pt, np.arange(n_vis), 64), wl.index_dim, W.seed + 1, total)
    k_new = host(W.k_new)
    kraw[e0:n_vis] = k_new[:max(0, n_vis - e0)]
    x_new = host(W.x_new)
    comp = O.compress_blocks(x_new, ctx, 4, host(W.gate_w), host(W.gate_b))

    def kv_fn(j):
        rows = regen_fill_rows(O.page_slot(pt, j, 64), 576, W.seed + 2, total).astype(np.float64)
        fresh = j >= e0
        rows[fresh] = comp[j[fresh] - e0]
        return rows

    xt = host(gen.device_normal((256, 576), W.seed + 3))  # positions ctx - 256 .. ctx - 1
    raw_rows = np.concatenate([xt, x_new[:t + 1]]).astype(np.float64)
    new_rows = np.arange(e0, n_vis)
    k_rope = (new_rows, 4 * new_rows + 3) if len(new_rows) else None
    return SeqState(wl, kraw, kv_fn, ctx - 256, raw_rows, host(W.q_idx[t]), host(W.w_idx[t]),
                    host(W.q_attn[t]), pos, n_vis, bands=bands, k_rope=k_rope)


def logical_of_phys(phys_row: np.ndarray, page_table_row: np.ndarray, page: int = 64) -> np.ndarray:
    """Logical entry j of each physical slot (-1 stays -1), through the
    inverse of the sequence's page table."""
    inv = {int(pg): i for i, pg in enumerate(page_table_row)}
    out = np.full(phys_row.shape, -1, dtype=np.int64)
    for k, s in enumerate(phys_row):
        if s >= 0:
            out[k] = inv[int(s) // page] * page + int(s) % page
    return out


def topk_agrees(o_logits: np.ndarray, got_logical: np.ndarray, k: int, tol):
    """The library's selection against the oracle's logits: k distinct entries
    (or all of them when fewer), equal to the oracle's top-k except for
    entries whose logit lies within tol of the k-th largest, where either
    choice is correct. tol is a scalar or per entry (then an entry is in the
    band when |logit - s_k| <= its tol + the k-th entry's tol).
    Returns (ok, sets_equal, n_in_band)."""
    n = len(o_logits)
    kk = min(k, n)
    sel = got_logical[got_logical >= 0]
    if len(sel) != kk or len(np.unique(sel)) != kk or sel.min() < 0 or sel.max() >= n:
        return False, False, 0
    want = O.topk_logical(o_logits, n, k)
    if kk == n:
        return bool(np.array_equal(np.sort(sel), want)), True, 0
    order = np.lexsort((np.arange(n), -o_logits))
    s_k = o_logits[order[kk - 1]]
    tol = np.broadcast_to(np.asarray(tol, dtype=np.float64), o_logits.shape)
    band = np.abs(o_logits - s_k) <= tol + tol[order[kk - 1]]
    a = np.zeros(n, bool)
    a[want] = True
    g = np.zeros(n, bool)
    g[sel] = True
    ok = np.array_equal(a & ~band, g & ~band)
    return bool(ok), bool(np.array_equal(a, g)), int(band.sum())
