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
        self.seed = seed  # base of every draw below (fills use seed*1000 + chunk)
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
        self.with_compress = with_compress
        self.x_new = gen.device_normal((B * 4, 576), seed + 4)  # the last 4 raw rows (token last)
        self.k_new = gen.device_normal((B, wl.index_dim), seed + 5)  # index-K row of that block
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
        # the caller's RoPE table over every position of the batch (the step's
        # index-K row and queries are rotated at the token's position)
        self.rope_table = None
        self.prep_flags = csa.CSA_PREP_HADAMARD if wl.hadamard else 0
        if wl.rope_dim:
            self.rope_table = torch.from_numpy(gen.rope_table(int(self.lens.max()), wl.rope_dim)).to(DEV)
            self.prep_flags |= csa.CSA_PREP_ROPE
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
        n = csa.csa_workspace_size(csa.CSA_OP_INDEXER_TOPK, B, self.maxN, wl.index_heads)
        self.itk_ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=DEV)  # counters start at 0
        torch.cuda.synchronize()

    def scan_plan(self):
        """(selects on chip, scan chunks per row) of indexer_topk512 at these
        sizes, by the library's rule: the scan chunk is about 1/256 of all
        entries, rounded up to 512, within [512, 4096]; the scan workgroups
        select their chunk's top-512 when a row has at most 256 chunks (more
        than 32 are merged into 8 lists before the final pass) and the rows
        do not take the row-block kernel (256 rows or more)."""
        chunk = min(4096, max(512, -(-(self.B * self.maxN // 256) // 512) * 512))
        chunks = -(-self.maxN // chunk)
        return chunks <= 256 and self.B < 256, chunks

    @property
    def indexer_kernel(self) -> str:
        fused, _ = self.scan_plan()
        fp4 = "true" if self.fmt == csa.CSA_MXFP4 else "false"
        if fused and self.B <= 256 and self.B * self.maxN > 256 * 4096:
            # more entries than 256 chunks of 4096: chunks planned on the device
            return f"indexer_wide_kernel<{fp4}>"
        return f"indexer_mfma_kernel<{fp4}, true, {'true' if fused else 'false'}>"

    def indexer_bytes(self) -> int:
        """Algorithmic bytes of one indexer scan launch: what the definition
        reads (index-K rows and scales of every visible entry, the prepared
        queries and their scales, the head weights, the page-table rows). The
        scan's own intermediates (the chunks' top-512 candidates on the fused
        path) are not counted."""
        per_entry = (self.wl.index_dim + 4) if self.fmt == csa.CSA_FP8_E4M3 else (self.wl.index_dim // 2 + 4)
        n = int(self.N.sum())
        q = self.B * self.wl.index_heads * (self.q_codes.shape[-1] + 4 + 4)
        return n * per_entry + q + n // C4_PAGE * 4

    def step_bytes(self) -> int:
        """Algorithmic bytes of a whole decode step: the indexer's inputs, the
        selection written (512 slots per query), the attention's gathers
        (selected + window entries, 644 B each) plus its q and output, and the
        step's cache writes and query preparation (the block's 4 raw rows read,
        the compressed entry, the token and the index-K row written; the raw
        index q read and prepared)."""
        ent = 644
        sel = self.B * 512 * 4
        att = self.B * (512 + self.wl.window) * ent + self.q_attn.numel() * 2 + self.out.numel() * 2
        comp = self.x_new.numel() * 2 + self.B * ent + self.B * ent
        krow = (self.wl.index_dim + 4) if self.fmt == csa.CSA_FP8_E4M3 else (self.wl.index_dim // 2 + 4)
        prep = (self.k_new.numel() * 2 + self.q_idx.numel() * 2
                + self.B * krow * (1 + self.wl.index_heads))
        return self.indexer_bytes() + sel + att + comp + prep

    def score_only(self, c: int):
        """The indexer logits of the step's rows into self.logits (indexer_score:
        the scan the step runs, writing logits instead of selecting on chip).
        For tests; run after step(c), whose preparation it reuses."""
        csa.indexer_score(self.q_codes, self.w_idx, self.row_seq, self.row_len, self.maxN, self.pt,
                          self.index_pools[c], self.logits, q_fmt=self.fmt, q_scale=self.q_scale)

    def step(self, c: int, ev=None):
        idx, kv = self.index_pools[c], self.c4_pools[c]
        wl = self.wl
        if self.with_compress:
            # the current token: compress the block it completes (L % 4 == 0),
            # append it to the raw window pool, prepare that block's index-K
            # row, and prepare the queries -- one launch
            csa.csa_decode_prep(self.x_new.view(self.B, 4, 576), self.q_pos, self.gate_w,
                                self.gate_b, self.pt, kv, self.pt, self.raw, k_rows=self.k_new,
                                q_rows=self.q_idx, kpool=idx, q_out=self.q_codes,
                                q_out_scale=self.q_scale, flags=self.prep_flags,
                                rope_table=self.rope_table)
        else:
            csa.csa_index_prep(self.q_idx, wl.index_dim, self.prep_flags, self.fmt,
                               self.q_codes, self.q_scale, rope_pos=self.q_pos,
                               rope_table=self.rope_table, rows_per_pos=wl.index_heads)
        if ev is not None:
            ev[0].record()
        # indexer + top-512 in one call: the scan workgroups select their
        # chunks' candidates on chip (the logits are not written), then one
        # final pass per row; ev[1] marks the end of the scan
        csa.indexer_topk512(self.q_codes, self.w_idx, self.row_seq, self.row_len, self.maxN, self.pt,
                            idx, self.phys, q_fmt=self.fmt, q_scale=self.q_scale, ws=self.itk_ws,
                            scan_done=None if ev is None else ev[1])
        csa.csa_sparse_attn(self.q_attn, self.row_seq, self.q_pos, self.phys, kv, self.raw, self.pt,
                            wl.window, wl.softmax_scale, self.out, ws=self.attn_ws)


class CsaSpecDecode(CsaDecode):
    """One multi-token (speculative-verify) decode step: each of B sequences
    of raw length L gains q_len = 4 tokens (positions L-4 .. L-1, one complete
    C4 block, L % 4 == 0) and runs q_len query rows. The cache writes are the
    block's compressed entry and index-K row and the four raw rows; each query
    row has its causal row length min(N, (p+1)/4) and its own window; the
    indexer gets the rows-per-sequence hint, so each index-K page is read once
    per sequence, not once per row."""

    def __init__(self, wl: Workload, lens, copies: int = 3, pool_pages: int | None = None):
        super().__init__(wl, lens, copies=copies, pool_pages=pool_pages)
        assert wl.q_len == 4 and all(int(L) % 4 == 0 for L in self.lens)
        B, Q, H = self.B, wl.q_len, self.H
        self.T = T = B * Q
        seed = self.seed
        pos = np.concatenate([np.arange(int(L) - Q, int(L)) for L in self.lens])
        self.pos_host = pos
        self.rows_len_host = np.minimum(np.repeat(self.N, Q), (pos + 1) // 4)
        self.row_seq = _i32(np.repeat(np.arange(B), Q))
        self.row_len = _i32(self.rows_len_host)
        self.q_pos = _i32(pos)
        self.last_pos = _i32(self.lens - 1)
        # the block's first three rows go to the raw pool in a ratio-1 store
        self.x_early = self.x_new.view(B, 4, 576)[:, :3].contiguous()
        self.early_cu = _i32(np.arange(B + 1) * 3)
        self.early_start = _i32(self.lens - 4)
        self.q_idx = gen.device_normal((T, wl.index_heads, wl.index_dim), seed + 16)
        self.w_idx = gen.device_uniform((T, wl.index_heads), seed + 17)
        self.q_attn = gen.device_normal((T, H, 576), seed + 18)
        self.phys = torch.empty((T, 512), dtype=torch.int32, device=DEV)
        self.out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=DEV)
        n = csa.csa_workspace_size(csa.CSA_OP_CSA_ATTN, T, 512 + wl.window, H)
        self.attn_ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        n = csa.csa_workspace_size(csa.CSA_OP_INDEXER_TOPK, T, self.maxN, wl.index_heads)
        self.itk_ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=DEV)
        qbytes = wl.index_dim if self.fmt == csa.CSA_FP8_E4M3 else wl.index_dim // 2
        self.q_codes = torch.empty((T, wl.index_heads, qbytes), dtype=torch.uint8, device=DEV)
        if self.fmt == csa.CSA_FP8_E4M3:
            self.q_scale = torch.empty((T, wl.index_heads), dtype=torch.float32, device=DEV)
        else:
            self.q_scale = torch.empty((T, wl.index_heads, wl.index_dim // 32), dtype=torch.uint8,
                                       device=DEV)
        self.zero_w, self.zero_b = torch.zeros(576, device=DEV), torch.zeros(1, device=DEV)
        self.logits = torch.empty((T, self.maxN), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()

    @property
    def indexer_kernel(self) -> str:
        fp4 = "true" if self.fmt == csa.CSA_MXFP4 else "false"
        return f"indexer_rows_kernel<{fp4}, {self.wl.q_len}, false>"

    def indexer_bytes(self) -> int:
        """Algorithmic bytes of the indexer launch: index-K rows of each
        sequence once (shared by its rows), the prepared queries and head
        weights, page-table rows and the logits written (this kernel's output
        is the logits, which the top-512 pass then reads)."""
        per_entry = (self.wl.index_dim + 4) if self.fmt == csa.CSA_FP8_E4M3 else (self.wl.index_dim // 2 + 4)
        n = int(self.N.sum())
        q = self.T * self.wl.index_heads * (self.wl.index_dim + 4 + 4)
        return n * per_entry + q + n // C4_PAGE * 4 + int(self.rows_len_host.sum()) * 4

    def step_bytes(self) -> int:
        """Algorithmic bytes of the multi-token step: the indexer launch (with
        its logits), the top-512 reading those logits and writing 512 slots per
        row, the attention's gathers, q and output per row, and the cache
        writes and query preparation."""
        ent = 644
        T = self.T
        topk = int(self.rows_len_host.sum()) * 4 + T * 512 * 4
        att = T * (512 + self.wl.window) * ent + self.q_attn.numel() * 2 + self.out.numel() * 2
        comp = self.x_new.numel() * 2 + self.B * ent + self.B * 4 * ent
        krow = (self.wl.index_dim + 4) if self.fmt == csa.CSA_FP8_E4M3 else (self.wl.index_dim // 2 + 4)
        prep = (self.k_new.numel() * 2 + self.q_idx.numel() * 2
                + (self.B + T * self.wl.index_heads) * krow)
        return self.indexer_bytes() + topk + att + comp + prep

    def score_only(self, c: int):
        """The step's indexer logits into self.logits (the same kernel as the
        step: indexer_score with the hint). For tests; run after step(c)."""
        csa.indexer_score(self.q_codes, self.w_idx, self.row_seq, self.row_len, self.maxN, self.pt,
                          self.index_pools[c], self.logits, q_fmt=self.fmt, q_scale=self.q_scale,
                          prep=csa.CSA_ROWS_PER_SEQ(self.wl.q_len))

    def step(self, c: int, ev=None):
        idx, kv = self.index_pools[c], self.c4_pools[c]
        wl = self.wl
        # the block the four tokens complete (compressed entry, index-K row) and
        # the last token's raw row, then the three earlier raw rows
        csa.csa_decode_prep(self.x_new.view(self.B, 4, 576), self.last_pos, self.gate_w, self.gate_b,
                            self.pt, kv, self.pt, self.raw, k_rows=self.k_new, kpool=idx,
                            flags=self.prep_flags, rope_table=self.rope_table)
        csa.c4_compress(self.x_early, self.early_cu, self.early_start, 3, 1, self.zero_w, self.zero_b,
                        self.pt, self.raw)
        csa.csa_index_prep(self.q_idx, wl.index_dim, self.prep_flags, self.fmt, self.q_codes,
                           self.q_scale, rope_pos=self.q_pos, rope_table=self.rope_table,
                           rows_per_pos=wl.index_heads)
        if ev is not None:
            ev[0].record()
        # the hint routes each sequence's four rows to one page walk
        csa.indexer_topk512(self.q_codes, self.w_idx, self.row_seq, self.row_len, self.maxN, self.pt,
                            idx, self.phys, q_fmt=self.fmt, q_scale=self.q_scale,
                            prep=csa.CSA_ROWS_PER_SEQ(wl.q_len), ws=self.itk_ws,
                            scan_done=None if ev is None else ev[1])
        csa.csa_sparse_attn(self.q_attn, self.row_seq, self.q_pos, self.phys, kv, self.raw, self.pt,
                            wl.window, wl.softmax_scale, self.out, ws=self.attn_ws)


class CsaPrefill:
    """Chunked prefill: `new` query tokens appended to a context of `ctx` raw
    tokens (batch 1). One step: compress the new tokens' blocks and append
    them to the raw pool, prepare their index-K rows, prepare every query's
    indexer q, score with the causal rule 4j+3 <= p, select per query, attend."""

    def __init__(self, wl: Workload, copies: int = 1):
        self.wl = wl
        new = wl.new_tokens
        L = wl.seq_len
        ctx = L - new
        self.ctx, self.new, self.L = ctx, new, L
        self.N = N = L // 4
        g = gen.rng(wl.seed)
        pages = L // RAW_PAGE
        self.P = P = pages
        pt = g.permutation(P).astype(np.int32)[None]
        self.pt_host = pt
        self.pt = _i32(pt)
        fmt = _FMT[wl.index_fmt]
        self.fmt = fmt
        seed = wl.seed * 10
        self.seed = seed
        self.idx = csa.alloc_index_pool(P, C4_PAGE, wl.index_dim, fmt, poison=False)
        fill_index_pool(self.idx, seed + 1, hadamard=wl.hadamard)
        self.c4 = csa.alloc_kv_pool(P, C4_PAGE, csa.CSA_FP8_E4M3, poison=False)
        fill_kv_pool_physical(self.c4, seed + 2)
        self.raw = csa.alloc_kv_pool(P, RAW_PAGE, csa.CSA_FP8_E4M3, poison=True)
        w0, b0 = torch.zeros(576, device=DEV), torch.zeros(1, device=DEV)
        self.zero_w, self.zero_b = w0, b0
        xt = gen.device_normal((RAW_PAGE, 576), seed + 3)  # context tail (window of the first queries)
        csa.c4_compress(xt, _i32([0, RAW_PAGE]), _i32([ctx - RAW_PAGE]), RAW_PAGE, 1, w0, b0, self.pt,
                        self.raw)
        gw, gb = gen.gate_params(g, 4)
        self.gate_w, self.gate_b = torch.from_numpy(gw).to(DEV), torch.from_numpy(gb).to(DEV)
        self.x_new = gen.device_normal((new, 576), seed + 4)
        self.cu_new, self.start_new = _i32([0, new]), _i32([ctx])
        nk = new // 4
        self.k_new = gen.device_normal((nk, wl.index_dim), seed + 5)
        ent = np.arange(ctx // 4, ctx // 4 + nk)
        self.k_dst = _i32(pt[0, ent // C4_PAGE] * C4_PAGE + ent % C4_PAGE)
        # RoPE: entry k's index-K row at the position that completes its block
        # (4k + 3), each query at its own position
        self.k_pos = _i32(4 * ent + 3)
        self.prep_flags = csa.CSA_PREP_HADAMARD if wl.hadamard else 0
        self.rope_table = None
        if wl.rope_dim:
            self.rope_table = torch.from_numpy(gen.rope_table(L, wl.rope_dim)).to(DEV)
            self.prep_flags |= csa.CSA_PREP_ROPE
        self.q_idx = gen.device_normal((new, wl.index_heads, wl.index_dim), seed + 6)
        self.w_idx = gen.device_uniform((new, wl.index_heads), seed + 7)
        self.q_attn = gen.device_normal((new, wl.heads, 576), seed + 8)
        self.q_codes = torch.empty((new, wl.index_heads, wl.index_dim), dtype=torch.uint8, device=DEV)
        self.q_scale = torch.empty((new, wl.index_heads), dtype=torch.float32, device=DEV)
        pos = ctx + np.arange(new)
        self.pos_host = pos
        self.row_len_host = np.minimum(N, (pos + 1) // 4)
        self.row_seq = _i32(np.zeros(new))
        self.row_len = _i32(self.row_len_host)
        self.q_pos = _i32(pos)
        self.phys = torch.empty((new, 512), dtype=torch.int32, device=DEV)
        self.out = torch.empty((new, wl.heads, 512), dtype=torch.bfloat16, device=DEV)
        n = csa.csa_workspace_size(csa.CSA_OP_CSA_ATTN, new, 512 + wl.window, wl.heads)
        self.attn_ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        # the fused indexer + top-512 (its workspace starts zero-filled)
        n = csa.csa_workspace_size(csa.CSA_OP_INDEXER_TOPK, new, N, wl.index_heads)
        self.itk_ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()

    def indexer_flops(self) -> float:
        """Causal indexer GEMM flops: 2 * heads * dim per visible (query, entry)."""
        return 2.0 * self.wl.index_heads * self.wl.index_dim * float(self.row_len_host.sum())

    def score_only(self, c: int = 0):
        """The step's indexer logits into self.logits (indexer_score: the same
        row-block kernel, writing logits instead of selecting on chip). For
        tests; run after step(c), whose preparation it reuses."""
        if getattr(self, "logits", None) is None:
            self.logits = torch.empty((self.new, self.N), dtype=torch.float32, device=DEV)
        csa.indexer_score(self.q_codes, self.w_idx, self.row_seq, self.row_len, self.N, self.pt,
                          self.idx, self.logits, q_fmt=self.fmt, q_scale=self.q_scale)

    def step(self, c: int = 0, ev=None):
        wl = self.wl
        csa.c4_compress(self.x_new, self.cu_new, self.start_new, self.new, 4, self.gate_w,
                        self.gate_b, self.pt, self.c4)
        csa.c4_compress(self.x_new, self.cu_new, self.start_new, self.new, 1, self.zero_w,
                        self.zero_b, self.pt, self.raw)
        kd = self.idx.data.view(-1, self.idx.data.shape[-1])
        ks = self.idx.scale.view(kd.shape[0], -1)
        csa.csa_index_prep(self.k_new, wl.index_dim, self.prep_flags, self.fmt, kd, ks, self.k_dst,
                           rope_pos=self.k_pos, rope_table=self.rope_table, rows_per_pos=1)
        csa.csa_index_prep(self.q_idx, wl.index_dim, self.prep_flags, self.fmt, self.q_codes,
                           self.q_scale, rope_pos=self.q_pos, rope_table=self.rope_table,
                           rows_per_pos=wl.index_heads)
        # the row-block scan keeps each query row's top-512 as it scores (one
        # page range per row at this size: no logits and no second pass)
        if ev is not None:
            ev[0].record()
        csa.indexer_topk512(self.q_codes, self.w_idx, self.row_seq, self.row_len, self.N, self.pt,
                            self.idx, self.phys, q_fmt=self.fmt, q_scale=self.q_scale,
                            ws=self.itk_ws)
        if ev is not None:
            ev[1].record()
        csa.csa_sparse_attn(self.q_attn, self.row_seq, self.q_pos, self.phys, self.c4, self.raw,
                            self.pt, wl.window, wl.softmax_scale, self.out, ws=self.attn_ws)


class HcaCsaRagged:
    """One decode step of an HCA layer and a CSA layer over a ragged batch
    (raw lengths log-uniform in [lo, hi]); the two layers share the raw
    window pool and its page table."""

    def __init__(self, wl: Workload, copies: int = 3):
        self.wl = wl
        n, lo, hi = wl.ragged
        self.lens = gen.ragged_lengths(gen.rng(wl.seed), n, lo, hi)
        self.csa = CsaDecode(wl, self.lens, copies=copies, seed_offset=1)
        g = gen.rng(wl.seed + 2)
        R = wl.hca_ratio
        nh = self.lens // R
        hpages = [max(1, (int(x) + C4_PAGE - 1) // C4_PAGE) for x in nh]
        Ph = int(sum(hpages))
        perm = g.permutation(Ph).astype(np.int32)
        hpt = np.zeros((n, max(hpages)), np.int32)
        o = 0
        for b, k in enumerate(hpages):
            hpt[b, :k] = perm[o:o + k]
            o += k
        self.hpt_host = hpt
        self.hpt = _i32(hpt)
        self.Ph = Ph
        self.hca_seed = wl.seed * 10 + 9
        base = csa.alloc_kv_pool(Ph, C4_PAGE, csa.CSA_FP8_E4M3, poison=False)
        fill_kv_pool_physical(base, self.hca_seed)
        self.hca_pools = [base] + [clone_kv_pool(base) for _ in range(copies - 1)]
        self.q_hca = gen.device_normal((n, wl.heads, 576), wl.seed * 10 + 10)
        self.out_hca = torch.empty((n, wl.heads, 512), dtype=torch.bfloat16, device=DEV)
        self.max_len = int(self.lens.max())
        k = csa.csa_workspace_size(csa.CSA_OP_HCA_ATTN, n, self.max_len // R + wl.window, wl.heads)
        self.hca_ws = torch.empty(max(k, 1), dtype=torch.uint8, device=DEV)
        self.B = n
        torch.cuda.synchronize()

    def hca_bytes(self) -> int:
        """Entries streamed by the HCA layer (visible compressed + window), 644 B each."""
        vis = self.lens // self.wl.hca_ratio
        win = np.minimum(self.lens, self.wl.window)
        return int((vis + win).sum()) * 644 + self.q_hca.numel() * 2 + self.out_hca.numel() * 2

    def step(self, c: int = 0, ev=None):
        wl = self.wl
        csa.hca_dense_attn(self.q_hca, self.csa.row_seq, self.csa.q_pos, self.max_len, wl.hca_ratio,
                           self.hca_pools[c], self.hpt, self.csa.raw, self.csa.pt, wl.window,
                           wl.softmax_scale, self.out_hca, ws=self.hca_ws)
        self.csa.step(c, ev)


def hca_build_input(lens, seed: int):
    """Raw rows of every sequence (bf16), drawn on the device in chunks, with
    their cu_rows; for timing the R=128 cache build."""
    total = int(np.sum(lens))
    x = torch.empty((total, 576), dtype=torch.bfloat16, device=DEV)
    for i, r0 in enumerate(range(0, total, 1 << 20)):
        r1 = min(total, r0 + (1 << 20))
        x[r0:r1] = gen.device_normal((r1 - r0, 576), seed * 1000 + i)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return x, _i32(cu), _i32(np.zeros(len(lens)))


class TinyDecode:
    """The tiny all-fp32 CSA decode: batch 1, raw length 4096 compressed 4:1 to
    1024 entries (identity page table), 8 x 64 fp32 indexer, top-512 of 1024,
    16 heads over the 576-dim KV plus a 128-token window. The pools are built
    once (c4_compress of the seeded raw rows; the index-K rows stored as
    drawn); one step is the indexer, the top-512 and the attention."""

    def __init__(self, wl: Workload):
        self.wl = wl
        g = gen.rng(wl.seed)
        L = wl.seq_len
        N = L // 4
        self.B, self.L, self.N = 1, L, N
        self.lens = np.array([L], dtype=np.int64)
        x = gen.normal(g, (L, 576))
        gw, gb = gen.gate_params(g, 4)
        kraw = gen.normal(g, (N, wl.index_dim))
        self.q_idx = torch.from_numpy(gen.normal(g, (1, wl.index_heads, wl.index_dim))).to(DEV)
        self.w_idx = torch.from_numpy(gen.uniform(g, (1, wl.index_heads))).to(DEV)
        self.q = torch.from_numpy(gen.normal(g, (1, wl.heads, 576))).to(DEV)
        P = L // RAW_PAGE
        ident = _i32(np.arange(P)[None])
        self.pt = ident
        self.c4 = csa.alloc_kv_pool(P, C4_PAGE, csa.CSA_F32)
        self.raw = csa.alloc_kv_pool(P, RAW_PAGE, csa.CSA_F32)
        xd = torch.from_numpy(x).to(DEV)
        cu, st = _i32([0, L]), _i32([0])
        csa.c4_compress(xd, cu, st, L, 4, torch.from_numpy(gw).to(DEV), torch.from_numpy(gb).to(DEV),
                        ident, self.c4)
        csa.c4_compress(xd, cu, st, L, 1, torch.zeros(576, device=DEV), torch.zeros(1, device=DEV),
                        ident, self.raw)
        self.kpool = csa.alloc_index_pool(P, C4_PAGE, wl.index_dim, csa.CSA_F32)
        csa.csa_index_prep(torch.from_numpy(kraw).to(DEV), wl.index_dim, 0, csa.CSA_F32,
                           self.kpool.data.view(-1, wl.index_dim))
        self.row_seq = _i32([0])
        self.row_len = _i32([N])
        self.q_pos = _i32([L - 1])
        self.phys = torch.empty((1, 512), dtype=torch.int32, device=DEV)
        self.out = torch.empty((1, wl.heads, 512), dtype=torch.float32, device=DEV)
        n = csa.csa_workspace_size(csa.CSA_OP_INDEXER_TOPK, 1, N, wl.index_heads)
        self.itk_ws = torch.zeros(max(n, 1), dtype=torch.uint8, device=DEV)
        n = csa.csa_workspace_size(csa.CSA_OP_CSA_ATTN_F32, 1, 512 + wl.window, wl.heads)
        self.attn_ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        torch.cuda.synchronize()

    def step_bytes(self) -> int:
        """Index-K rows (fp32), q and weights, selected + window entries (fp32,
        576 dims), output."""
        wl = self.wl
        return (self.N * wl.index_dim * 4 + wl.index_heads * (wl.index_dim + 1) * 4
                + (512 + wl.window) * 576 * 4 + wl.heads * (576 + 512) * 4 + 512 * 4)

    def step(self, c: int = 0, ev=None):
        wl = self.wl
        if ev is not None:
            ev[0].record()
        csa.indexer_topk512(self.q_idx, self.w_idx, self.row_seq, self.row_len, self.N, self.pt,
                            self.kpool, self.phys, ws=self.itk_ws,
                            scan_done=None if ev is None else ev[1])
        csa.csa_sparse_attn(self.q, self.row_seq, self.q_pos, self.phys, self.c4, self.raw, self.pt,
                            wl.window, wl.softmax_scale, self.out, ws=self.attn_ws)
