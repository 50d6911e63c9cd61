"""End-to-end check of the tiny all-fp32 CSA decode (batch 1, raw length 4096,
C4 compression to 1024 entries, 8 x 64 indexer, top-512 of 1024, 16 heads,
128-token window, identity page table), HIP path against the oracle.

Both sides start from the same seeded raw draws. The compressed KV is
compared to 2e-5 relative; the logits to 1e-4 of the row max; the top-512
sets outside the near-tie band (|logit - s_512| <= 1e-3 |s_512|) must agree;
the attention output must be within 1e-4 of each head's max, against the
oracle's attention over the entries the GPU selected (the selection itself is
checked against the oracle's logits above; where several selections are
correct, the attention over the one taken must still be right).
Used by the GPU test suite and by the smoke check.
"""
from __future__ import annotations

import numpy as np

from oracle import csa_oracle as O
from workloads import gen, specs


def run_tiny_decode_check(csa, torch, seed_offset: int = 0) -> dict:
    wl = specs.TINY_FP32_DECODE
    dev = "cuda"
    g = gen.rng(wl.seed + seed_offset)
    L, N = wl.seq_len, wl.seq_len // 4
    x = gen.normal(g, (L, 576))
    gw, gb = gen.gate_params(g, 4)
    kraw = gen.normal(g, (N, wl.index_dim))
    q_idx = gen.normal(g, (1, wl.index_heads, wl.index_dim))
    w_idx = gen.uniform(g, (1, wl.index_heads))
    q = gen.normal(g, (1, wl.heads, 576))
    P = L // 256
    ident = np.arange(P, dtype=np.int32)[None]

    def T(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    c4 = csa.alloc_kv_pool(P, 64, csa.CSA_F32)
    raw = csa.alloc_kv_pool(P, 256, csa.CSA_F32)
    cu, st = T(np.array([0, L], np.int32)), T(np.array([0], np.int32))
    csa.c4_compress(T(x), cu, st, L, 4, T(gw), T(gb), T(ident), c4)
    csa.c4_compress(T(x), cu, st, L, 1, T(np.zeros(576, np.float32)), T(np.zeros(1, np.float32)),
                    T(ident), raw)
    kpool = csa.alloc_index_pool(P, 64, wl.index_dim, csa.CSA_F32)
    csa.csa_index_prep(T(kraw), wl.index_dim, 0, csa.CSA_F32, kpool.data.view(-1, wl.index_dim))
    logits = torch.full((1, N), float("nan"), device=dev)
    row = T(np.array([0], np.int32))
    nlen = T(np.array([N], np.int32))
    csa.indexer_score(T(q_idx), T(w_idx), row, nlen, N, T(ident), kpool, logits)
    phys = torch.empty((1, 512), dtype=torch.int32, device=dev)
    logical = torch.empty((1, 512), dtype=torch.int32, device=dev)
    csa.topk512_page_select(logits, nlen, row, T(ident), phys, logical)
    out = torch.empty((1, wl.heads, 512), dtype=torch.float32, device=dev)
    csa.csa_sparse_attn(T(q), row, T(np.array([L - 1], np.int32)), phys, c4, raw, T(ident),
                        wl.window, wl.softmax_scale, out)
    torch.cuda.synchronize()

    # oracle
    c = O.compress_blocks(x, 0, 4, gw, gb)
    c4_gpu = np.concatenate([c4.latent.cpu().numpy().reshape(-1, 512),
                             c4.rope.cpu().numpy().reshape(-1, 64)], axis=1)[:N]
    comp_err = float(np.max(np.abs(c4_gpu - c) / (np.abs(c) + 1e-3)))
    assert np.allclose(c4_gpu, c, rtol=2e-5, atol=2e-6), f"compressed KV differs ({comp_err})"
    o_logits = O.indexer_logits(q_idx[0], w_idx[0], kraw)
    g_logits = logits.cpu().numpy()[0]
    lerr = float(np.abs(g_logits - o_logits).max() / np.abs(o_logits).max())
    assert lerr <= 1e-4, f"logits differ ({lerr})"
    sel_o = O.topk_logical(o_logits, N)
    sel_g = np.sort(logical.cpu().numpy()[0])
    s512 = np.sort(o_logits)[::-1][511]
    band = np.abs(o_logits - s512) <= 1e-3 * abs(s512)
    outside = ~band
    assert np.array_equal(np.isin(np.arange(N), sel_o) & outside, np.isin(np.arange(N), sel_g) & outside)
    assert len(sel_g) == 512 and len(np.unique(sel_g)) == 512
    phys_ok = np.array_equal(phys.cpu().numpy()[0], logical.cpu().numpy()[0])  # identity table
    assert phys_ok
    res = {"compress_rel_err": comp_err, "logits_rel_err": lerr, "topk_equal": bool(np.array_equal(sel_o, sel_g))}
    # attention over the GPU's selection (identity page table: slot = entry)
    c4p = O.KVPool(*O.quant_kv_entries(c, "f32"), "f32")
    rawp = O.KVPool(*O.quant_kv_entries(x, "f32"), "f32")
    want = O.csa_attention_query(q[0], c4p.rows(sel_g), rawp.rows(O.window_positions(L - 1, wl.window)),
                                 wl.softmax_scale)
    got = out.cpu().numpy()[0]
    aerr = float((np.abs(got - want).max(axis=1) / np.abs(want).max(axis=1)).max())
    assert aerr <= 1e-4, f"attention differs ({aerr})"
    res["attn_rel_err"] = aerr
    return res
