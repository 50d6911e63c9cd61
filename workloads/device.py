"""Device-resident synthetic workloads for timing and full-size checks.

Raw values are seeded torch draws on the GPU (workloads.gen); the paged pools
are then built by the library's own entry points (csa_index_prep for
index-K rows, c4_compress with ratio 1 for KV entries), so this module holds
no arithmetic of the method itself. Several identical copies of the large
pools can be made so that consecutive timed steps read different memory and
the 256 MB last-level cache cannot serve a step from the previous one.
"""
from __future__ import annotations

import numpy as np
import torch

import compressed_sparse_attention_c4_amd as csa
from workloads import gen
from workloads.specs import C4_PAGE, RAW_PAGE, Workload

DEV = "cuda"
_FMT = {"fp8": csa.CSA_FP8_E4M3, "mxfp4": csa.CSA_MXFP4, "f32": csa.CSA_F32}
_CHUNK = 1 << 17


def _i32(a):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=DEV)


def fill_index_pool(pool: csa.IndexPool, seed: int, hadamard=True):
    """Every physical row <- rotate + quantise(N(0,1) bf16 draw)."""
    rows = pool.num_pages * pool.page_size
    data = pool.data.view(rows, -1)
    scale = pool.scale.view(rows, -1) if pool.scale is not None else None
    flags = csa.CSA_PREP_HADAMARD if hadamard else 0
    for i, r0 in enumerate(range(0, rows, _CHUNK)):
        r1 = min(rows, r0 + _CHUNK)
        v = gen.device_normal((r1 - r0, pool.dim), seed * 1000 + i)
        csa.csa_index_prep(v, pool.dim, flags, pool.fmt, data[r0:r1],
                           None if scale is None else scale[r0:r1])


def fill_kv_pool_physical(pool: csa.KvPool, seed: int):
    """Every physical slot <- quantised N(0,1) bf16 576-vector (ratio-1 store
    through an identity page table)."""
    slots = pool.num_pages * pool.page_size
    ident = _i32(np.arange(pool.num_pages)[None])
    w = torch.zeros(576, device=DEV)
    b = torch.zeros(1, device=DEV)
    for i, r0 in enumerate(range(0, slots, _CHUNK)):
        r1 = min(slots, r0 + _CHUNK)
        x = gen.device_normal((r1 - r0, 576), seed * 1000 + i)
        csa.c4_compress(x, _i32([0, r1 - r0]), _i32([r0]), r1 - r0, 1, w, b, ident, pool)


def clone_index_pool(p: csa.IndexPool) -> csa.IndexPool:
    return csa.IndexPool(p.data.clone(), None if p.scale is None else p.scale.clone(), p.fmt, p.dim,
                         p.page_size)


def clone_kv_pool(p: csa.KvPool) -> csa.KvPool:
    return csa.KvPool(p.latent.clone(), None if p.scale is None else p.scale.clone(), p.rope.clone(),
                      p.fmt, p.page_size)


class CsaDecode:
    """One CSA decode step for a batch of sequences of raw lengths `lens`
    (the current token is the last raw token, p = L - 1)."""

    def __init__(self, wl: Workload, lens, copies: int = 3, pool_pages: int | None = None,
                 seed_offset: int = 0, with_compress: bool = True):
        self.wl = wl
        self.B = B = len(lens)
        self.lens = np.asarray(lens, dtype=np.int64)
        self.N = self.lens // 4
        self.H = wl.heads
        g = gen.rng(wl.seed + seed_offset)
        pages = [(int(L) + RAW_PAGE - 1) // RAW_PAGE for L in self.lens]  # = ceil(N / 64)
        pps = max(pages)
        need = int(sum(pages))
        P = max(pool_pages or need, need)
        perm = g.permutation(P).astype(np.int32)
        pt = np.zeros((B, pps), np.int32)
        o = 0
        for b, n in enumerate(pages):
            pt[b, :n] = perm[o:o + n]
            o += n
        self.pt_host = pt
        self.pt = _i32(pt)
        self.P = P
        fmt = _FMT[wl.index_fmt]
        seed = wl.seed * 10 + seed_offset
        base_idx = csa.alloc_index_pool(P, C4_PAGE, wl.index_dim, fmt, poison=False)
        fill_index_pool(base_idx, seed + 1, hadamard=wl.hadamard)
        base_kv = csa.alloc_kv_pool(P, C4_PAGE, csa.CSA_FP8_E4M3, poison=False)
        fill_kv_pool_physical(base_kv, seed + 2)
        self.index_pools = [base_idx] + [clone_index_pool(base_idx) for _ in range(copies - 1)]
        self.c4_pools = [base_kv] + [clone_kv_pool(base_kv) for _ in range(copies - 1)]
        # raw pool shares the page table (256 raw tokens per page); only the
        # last two pages of each sequence (the window) are written
        self.raw = csa.alloc_kv_pool(P, RAW_PAGE, csa.CSA_FP8_E4M3, poison=True)
        tail = 2 * RAW_PAGE
        starts = np.maximum(self.lens - tail, 0)
        nrows = self.lens - starts
        cu = np.concatenate([[0], np.cumsum(nrows)])
        x = gen.device_normal((int(cu[-1]), 576), seed + 3)
        w0, b0 = torch.zeros(576, device=DEV), torch.zeros(1, device=DEV)
        csa.c4_compress(x, _i32(cu), _i32(starts), int(nrows.max()), 1, w0, b0, self.pt, self.raw)
        # step inputs
        gw, gb = gen.gate_params(g, 4)
        self.gate_w, self.gate_b = torch.from_numpy(gw).to(DEV), torch.from_numpy(gb).to(DEV)
        self.zero_w, self.zero_b = w0, b0  # ratio-1 store of the raw token
        self.with_compress = with_compress
        self.x_new = gen.device_normal((B * 4, 576), seed + 4)          # last block's raw rows
        self.x_tok = self.x_new.view(B, 4, 576)[:, 3].contiguous()      # the current token
        self.cu_new = _i32(np.arange(0, 4 * B + 1, 4))
        self.start_new = _i32(self.lens - 4)
        self.cu_tok = _i32(np.arange(B + 1))
        self.start_tok = _i32(self.lens - 1)
        self.k_new = gen.device_normal((B, wl.index_dim), seed + 5)
        last = self.N - 1
        self.k_dst = _i32(pt[np.arange(B), last // C4_PAGE] * C4_PAGE + last % C4_PAGE)
        self.q_idx = gen.device_normal((B, wl.index_heads, wl.index_dim), seed + 6)
        self.w_idx = gen.device_uniform((B, wl.index_heads), seed + 7)
        self.q_attn = gen.device_normal((B, self.H, 576), seed + 8)
        qbytes = wl.index_dim if fmt == csa.CSA_FP8_E4M3 else wl.index_dim // 2
        self.q_codes = torch.empty((B, wl.index_heads, qbytes), dtype=torch.uint8, device=DEV)
        if fmt == csa.CSA_FP8_E4M3:
            self.q_scale = torch.empty((B, wl.index_heads), dtype=torch.float32, device=DEV)
        else:
            self.q_scale = torch.empty((B, wl.index_heads, wl.index_dim // 32), dtype=torch.uint8, device=DEV)
        self.fmt = fmt
        self.maxN = int(self.N.max())
        self.logits = torch.empty((B, self.maxN), dtype=torch.float32, device=DEV)
        self.row_seq = _i32(np.arange(B))
        self.row_len = _i32(self.N)
        self.q_pos = _i32(self.lens - 1)
        self.phys = torch.empty((B, 512), dtype=torch.int32, device=DEV)
        self.out = torch.empty((B, self.H, 512), dtype=torch.bfloat16, device=DEV)
        n = csa.csa_workspace_size(csa.CSA_OP_CSA_ATTN, B, 512 + wl.window, self.H)
        self.attn_ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        n = csa.csa_workspace_size(csa.CSA_OP_TOPK, B, self.maxN, 1)
        self.topk_ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()

    # algorithmic bytes of one indexer launch: index-K rows + prepared q +
    # head weights + page-table rows + logits written
    def indexer_bytes(self) -> int:
        per_entry = (self.wl.index_dim + 4) if self.fmt == csa.CSA_FP8_E4M3 else (self.wl.index_dim // 2 + 4)
        n = int(self.N.sum())
        q = self.B * self.wl.index_heads * (self.q_codes.shape[-1] + 4 + 4)
        return n * per_entry + q + n // C4_PAGE * 4 + n * 4

    def step_bytes(self) -> int:
        """Algorithmic bytes of a whole step: indexer, top-k read of the logits
        and writes of 512 indices, attention gathers (selected + window
        entries, 644 B each) plus q and output, compress / prep writes."""
        ent = 644
        att = self.B * (512 + self.wl.window) * ent + self.q_attn.numel() * 2 + self.out.numel() * 2
        topk = int(self.N.sum()) * 4 + self.B * 512 * 4
        comp = self.x_new.numel() * 2 + self.B * ent + self.x_tok.numel() * 2 + self.B * ent
        prep = self.k_new.numel() * 2 + self.q_idx.numel() * 2 + self.B * 132 * (1 + self.wl.index_heads)
        return self.indexer_bytes() + topk + att + comp + prep

    def step(self, c: int, ev=None):
        idx, kv = self.index_pools[c], self.c4_pools[c]
        wl = self.wl
        if self.with_compress:
            # the current token completes block N-1: compress it, append the
            # token to the raw window pool, prepare its index-K row
            csa.c4_compress(self.x_new, self.cu_new, self.start_new, 4, 4, self.gate_w, self.gate_b,
                            self.pt, kv)
            csa.c4_compress(self.x_tok, self.cu_tok, self.start_tok, 1, 1, self.zero_w, self.zero_b,
                            self.pt, self.raw)
            kd = idx.data.view(-1, idx.data.shape[-1])
            ks = idx.scale.view(kd.shape[0], -1)
            csa.csa_index_prep(self.k_new, wl.index_dim, csa.CSA_PREP_HADAMARD, self.fmt, kd, ks,
                               self.k_dst)
        csa.csa_index_prep(self.q_idx, wl.index_dim, csa.CSA_PREP_HADAMARD, self.fmt, self.q_codes,
                           self.q_scale)
        if ev is not None:
            ev[0].record()
        csa.indexer_score(self.q_codes, self.w_idx, self.row_seq, self.row_len, self.maxN, self.pt,
                          idx, self.logits, q_fmt=self.fmt, q_scale=self.q_scale)
        if ev is not None:
            ev[1].record()
        csa.topk512_page_select(self.logits, self.row_len, self.row_seq, self.pt, self.phys,
                                ws=self.topk_ws)
        csa.csa_sparse_attn(self.q_attn, self.row_seq, self.q_pos, self.phys, kv, self.raw, self.pt,
                            wl.window, wl.softmax_scale, self.out, ws=self.attn_ws)
