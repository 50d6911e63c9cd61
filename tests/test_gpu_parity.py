"""GPU parity: each entry point of libcsa.so against the CPU oracle on the same
seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles / pages and a ragged tail.

Bars: index and selection work bit-exact; quantised codes equal except a
one-code step where the oracle's fp32 pre-rounding value sits within 1e-5 of
the midpoint (two correct fp32 evaluations may round apart there); logits
within 1e-4 of the row's max magnitude; attention within 1e-4 (relative to
the row's max) for the fp32 path and 2e-2 max-abs for the bf16 / FP8 path.
"""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_helpers import (DEV, fp8_codes_match, index_pool_to_device, kv_pool_to_device,
                               t_dev, unpack_e2m1)
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_c4_amd as m
    return m


def _bf16(x):
    """float32 array -> (torch bf16 device tensor, float32 host values it holds)."""
    bits = gen.to_bf16_bits(x)
    return t_dev(bits.view(np.int16)).view(torch.bfloat16), gen.bf16_bits_to_f32(bits)


# ------------------------------------------------------------------ index prep


@pytest.mark.parametrize("rows", [1, 77, 3000])
def test_index_prep_fp8_hadamard(csa, rows):
    g = gen.rng(100 + rows)
    v, vh = _bf16(gen.normal(g, (rows, 128)))
    out = torch.full((rows, 128), 0xAB, dtype=torch.uint8, device=DEV)
    sc = torch.empty(rows, dtype=torch.float32, device=DEV)
    csa.csa_index_prep(v, 128, csa.CSA_PREP_HADAMARD, csa.CSA_FP8_E4M3, out, sc)
    codes, scale = O.index_prep(vh, True, "fp8")
    # the decision is taken on the same float32 butterfly values: bit-exact
    assert np.array_equal(sc.cpu().numpy(), scale)
    assert np.array_equal(out.cpu().numpy(), codes)


@pytest.mark.parametrize("rows", [5, 1000])
def test_index_prep_mxfp4_hadamard(csa, rows):
    g = gen.rng(200 + rows)
    v, vh = _bf16(gen.normal(g, (rows, 128)))
    out = torch.empty((rows, 64), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows, 4), dtype=torch.uint8, device=DEV)
    csa.csa_index_prep(v, 128, csa.CSA_PREP_HADAMARD, csa.CSA_MXFP4, out, sc)
    codes, sbytes = O.index_prep(vh, True, "mxfp4")
    assert np.array_equal(sc.cpu().numpy(), sbytes)
    assert np.array_equal(out.cpu().numpy(), codes)


def test_index_prep_f32_dst_rows(csa):
    """Rows go to dst_rows[i]; a negative destination skips the row."""
    g = gen.rng(300)
    v = gen.normal(g, (50, 64))
    dst = np.random.default_rng(1).permutation(80)[:50].astype(np.int32)
    dst[[3, 17, 49]] = -1
    out = torch.full((80, 64), float("nan"), dtype=torch.float32, device=DEV)
    csa.csa_index_prep(t_dev(v), 64, csa.CSA_PREP_HADAMARD, csa.CSA_F32, out, None, t_dev(dst))
    want = O.hadamard_rotate_f32(v)
    got = out.cpu().numpy()
    keep = dst >= 0
    assert np.array_equal(got[dst[keep]], want[keep])
    untouched = np.setdiff1d(np.arange(80), dst[keep])
    assert np.all(np.isnan(got[untouched]))


# ------------------------------------------------------------------ compressor


def _compress_case(csa, ratio, fmt, seqs, rows_per_seq, starts, seed):
    g = gen.rng(seed)
    w, b = gen.gate_params(g, ratio)
    xs = [gen.normal(g, (n, 576)) for n in rows_per_seq]
    x, xh = _bf16(np.concatenate(xs))
    cu = np.concatenate([[0], np.cumsum(rows_per_seq)]).astype(np.int32)
    ps = 64
    blocks = [(s + n) // ratio for s, n in zip(starts, rows_per_seq)]
    pages_per_seq = max(blocks) // ps + 2
    num_pages = seqs * pages_per_seq + 3
    pt = gen.page_table(g, seqs, pages_per_seq, num_pages)
    out = csa.alloc_kv_pool(num_pages, ps, csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_F32)
    csa.c4_compress(x, t_dev(cu), t_dev(np.array(starts, np.int32)), max(rows_per_seq), ratio,
                    t_dev(w), t_dev(b), t_dev(pt), out)
    torch.cuda.synchronize()
    return g, w, b, xh, cu, pt, out


@pytest.mark.parametrize("ratio,rows,starts", [
    (4, [4096, 37, 4], [0, 8, 4096]),          # several pages, ragged tail, single block
    (128, [2000, 128 * 3 + 5], [0, 1024]),     # HCA ratio
    (1, [300], [100]),                         # raw-token append
])
def test_compress_f32_pool(csa, ratio, rows, starts):
    g, w, b, xh, cu, pt, out = _compress_case(csa, ratio, "f32", len(rows), rows, starts, 400 + ratio)
    lat = out.latent.cpu().numpy().reshape(-1, 512)
    rope = out.rope.cpu().numpy().reshape(-1, 64)
    written = np.zeros(lat.shape[0], bool)
    for s in range(len(rows)):
        want = O.compress_blocks(xh[cu[s]:cu[s + 1]], starts[s], ratio, w, b)
        kb0 = starts[s] // ratio
        slots = O.page_slot(pt[s], np.arange(kb0, kb0 + len(want)), 64)
        got = np.concatenate([lat[slots], rope[slots]], axis=1)
        np.testing.assert_allclose(got, want, rtol=2e-5, atol=2e-6)
        written[slots] = True
    assert np.all(np.isnan(lat[~written])), "compress wrote outside its blocks"


@pytest.mark.parametrize("ratio", [4, 128])
def test_compress_fp8_pool(csa, ratio):
    rows = [4096 + 13, 1000]
    starts = [0, 256]
    g, w, b, xh, cu, pt, out = _compress_case(csa, ratio, "fp8", 2, rows, starts, 500 + ratio)
    lat = out.latent.cpu().numpy().reshape(-1, 512)
    sc = out.scale.cpu().numpy().reshape(-1)
    rope = out.rope.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1, 64)
    total_bad = 0
    for s in range(2):
        c = O.compress_blocks(xh[cu[s]:cu[s + 1]], starts[s], ratio, w, b)
        ocodes, oscale, orope = O.quant_kv_entries(c, "fp8")
        kb0 = starts[s] // ratio
        slots = O.page_slot(pt[s], np.arange(kb0, kb0 + len(c)), 64)
        # scales agree to fp32 rounding of amax of two fp32 evaluations of c
        np.testing.assert_allclose(sc[slots], oscale, rtol=3e-6)
        ratio_o = c[:, :512].astype(np.float32) / oscale[:, None]
        ok, nbad = fp8_codes_match(lat[slots], ocodes, ratio_o, rel=2e-5)
        assert ok
        total_bad += nbad
        # bf16 RoPE dims: one bf16 rounding of two fp32 evaluations of c
        gr, orr = O.bf16_decode(rope[slots]), O.bf16_decode(orope)
        assert np.all(np.abs(gr - orr) <= 2.0 ** -7 * np.abs(orr) + 1e-5)
    assert total_bad <= 20


# ------------------------------------------------------------------ indexer


def _index_case(g, fmt, seqs, lens, H=64, D=128, ps=64, extra_pages=5):
    pages = [(n + ps - 1) // ps for n in lens]
    pps = max(pages)
    num_pages = seqs * pps + extra_pages
    pt = gen.page_table(g, seqs, pps, num_pages)
    kraw = gen.normal(g, (num_pages * ps, D))
    data, sc = O.index_prep(kraw, fmt != "f32", fmt)
    pool = O.IndexPool(data, sc, fmt)
    return pt, pool, num_pages


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_indexer_prepared_query(csa, fmt):
    """Both sides score the same stored bytes: logits within 1e-4 of row max."""
    g = gen.rng(600 + len(fmt))
    lens = [5000, 513, 64 * 7 + 3, 17]
    pt, pool, num_pages = _index_case(g, fmt, len(lens), lens)
    qraw = gen.normal(g, (len(lens), 64, 128))
    qcodes, qsc = O.index_prep(qraw, True, fmt)
    w = gen.uniform(g, (len(lens), 64))
    ld = 5008
    logits = torch.full((len(lens), ld), float("nan"), device=DEV)
    dpool = index_pool_to_device(pool, 64, 128)
    qfmt = csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_MXFP4
    qs = t_dev(qsc.astype(np.float32)) if fmt == "fp8" else t_dev(qsc)
    csa.indexer_score(t_dev(qcodes), t_dev(w), t_dev(np.arange(len(lens), dtype=np.int32)),
                      t_dev(np.array(lens, np.int32)), max(lens), t_dev(pt), dpool, logits,
                      q_fmt=qfmt, q_scale=qs)
    got = logits.cpu().numpy()
    qhat = O.index_dequant(qcodes, qsc, fmt)
    for t, n in enumerate(lens):
        slots = O.page_slot(pt[t], np.arange(n), 64)
        want = O.indexer_logits(qhat[t], w[t], pool.rows(slots))
        np.testing.assert_allclose(got[t, :n], want, rtol=0, atol=1e-4 * np.abs(want).max())
        assert np.all(np.isnan(got[t, n:])), "wrote past row_len"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_indexer_fused_query_prep(csa, fmt):
    """bf16 query rotated and quantised inside the call: the prepared codes
    (q_used) match the oracle's, and the logits match where they do."""
    g = gen.rng(700 + len(fmt))
    lens = [3000, 1000]
    pt, pool, _ = _index_case(g, fmt, 2, lens)
    q, qh = _bf16(gen.normal(g, (2, 64, 128)))
    w = gen.uniform(g, (2, 64))
    logits = torch.full((2, 3000), float("nan"), device=DEV)
    if fmt == "fp8":
        qu = torch.empty((2, 64, 128), dtype=torch.uint8, device=DEV)
        qus = torch.empty((2, 64), dtype=torch.float32, device=DEV)
    else:
        qu = torch.empty((2, 64, 64), dtype=torch.uint8, device=DEV)
        qus = torch.empty((2, 64, 4), dtype=torch.uint8, device=DEV)
    csa.indexer_score(q, t_dev(w), t_dev(np.arange(2, dtype=np.int32)), t_dev(np.array(lens, np.int32)),
                      3000, t_dev(pt), index_pool_to_device(pool, 64, 128), logits,
                      prep=csa.CSA_PREP_HADAMARD | csa.CSA_PREP_QUANT, q_used=qu, q_used_scale=qus)
    qcodes, qsc = O.index_prep(qh, True, fmt)
    assert np.array_equal(qu.cpu().numpy(), qcodes)
    assert np.array_equal(qus.cpu().numpy(), qsc)
    qhat = O.index_dequant(qcodes, qsc, fmt)
    got = logits.cpu().numpy()
    for t, n in enumerate(lens):
        want = O.indexer_logits(qhat[t], w[t], pool.rows(O.page_slot(pt[t], np.arange(n), 64)))
        np.testing.assert_allclose(got[t, :n], want, rtol=0, atol=1e-4 * np.abs(want).max())


def test_indexer_f32(csa):
    g = gen.rng(800)
    lens = [1024, 700]
    pt, pool, _ = _index_case(g, "f32", 2, lens, H=8, D=64)
    q = gen.normal(g, (2, 8, 64))
    w = gen.uniform(g, (2, 8))
    logits = torch.full((2, 1024), float("nan"), device=DEV)
    csa.indexer_score(t_dev(q), t_dev(w), t_dev(np.arange(2, dtype=np.int32)),
                      t_dev(np.array(lens, np.int32)), 1024, t_dev(pt),
                      index_pool_to_device(pool, 64, 64), logits)
    got = logits.cpu().numpy()
    for t, n in enumerate(lens):
        want = O.indexer_logits(q[t], w[t], pool.rows(O.page_slot(pt[t], np.arange(n), 64)))
        np.testing.assert_allclose(got[t, :n], want, rtol=1e-5, atol=1e-5 * np.abs(want).max())


# ------------------------------------------------------------------ top-512


def _run_topk(csa, logits, lens, pt):
    R = len(lens)
    phys = torch.full((R, 512), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((R, 512), -7, dtype=torch.int32, device=DEV)
    csa.topk512_page_select(t_dev(logits.astype(np.float32)), t_dev(np.array(lens, np.int32)),
                            t_dev(np.arange(R, dtype=np.int32)), t_dev(pt), phys, logi)
    return phys.cpu().numpy(), logi.cpu().numpy()


@pytest.mark.parametrize("case", ["random", "ties", "short", "special", "long", "near_ties", "positive"])
def test_topk_bit_exact(csa, case):
    g = gen.rng(900 + len(case))
    if case == "random":
        lens = [32768, 4097, 513, 10000]
    elif case == "ties":
        lens = [20000, 3000]
    elif case == "short":
        lens = [0, 1, 511, 512, 100]
    elif case == "special":
        lens = [2000, 1500]
    elif case in ("near_ties", "positive"):
        lens = [32768, 5000, 600]
    else:
        lens = [262144]
    L = max(max(lens), 1)
    pps = (L + 63) // 64
    pt = gen.page_table(g, len(lens), pps, len(lens) * pps + 7)
    logits = g.standard_normal((len(lens), L)).astype(np.float32) * 10
    if case == "ties":
        logits = np.round(logits / 4) * 4  # few distinct values, heavy ties
    if case == "near_ties":  # equal values inside the threshold bucket, bucket fits in LDS
        logits = np.round(logits * 20) / 20
    if case == "positive":  # indexer-like: positive, crowded into few exponent buckets
        logits = np.abs(logits) * 3 + 200
    if case == "special":
        logits[0, ::3] = -0.0
        logits[0, 1::3] = 0.0
        logits[0, 5:900] = 0.0
        logits[1, :] = -np.inf
        logits[1, 100:300] = 1.0
        logits[1, 7] = np.nan
        logits[1, 1000] = np.inf
    phys, logi = _run_topk(csa, logits, lens, pt)
    for r, n in enumerate(lens):
        wp, wl = O.topk_page_select(logits[r], n, pt[r])
        assert np.array_equal(logi[r], wl), f"row {r}: logical indices differ"
        assert np.array_equal(phys[r], wp), f"row {r}: physical slots differ"


@pytest.mark.parametrize("R,L", [(130, 20000),   # chunks on 256-thread workgroups
                                 (128, 9000)])   # one workgroup per row, 16 keys per lane
def test_topk_many_rows(csa, R, L):
    """Batches of >= 128 rows take their own launch plan; rows of every kind
    (random, heavy ties, short, NaN / -inf / -0, all equal) in one batch."""
    g = gen.rng(950 + R)
    lens = g.integers(L // 2, L + 1, size=R)
    lens[:6] = [0, 1, 511, 512, 513, L]
    pps = (L + 63) // 64
    pt = gen.page_table(g, R, pps, R * pps + 3)
    logits = (g.standard_normal((R, L)) * 10).astype(np.float32)
    logits[6:20] = np.round(logits[6:20] / 4) * 4
    logits[20] = 1.5
    logits[21, ::2] = -np.inf
    logits[21, 3::7] = np.nan
    logits[22, ::3] = -0.0
    logits[22, 1::3] = 0.0
    logits[23:30] = np.abs(logits[23:30]) * 3 + 200
    phys, logi = _run_topk(csa, logits, lens.tolist(), pt)
    for r, n in enumerate(lens):
        wp, wl = O.topk_page_select(logits[r], int(n), pt[r])
        assert np.array_equal(logi[r], wl), f"row {r} (len {n}): logical indices differ"
        assert np.array_equal(phys[r], wp), f"row {r} (len {n}): physical slots differ"


def test_topk_identity_table_and_all_equal(csa):
    logits = np.full((1, 5000), 2.5, np.float32)
    pt = np.arange(79, dtype=np.int32)[None]
    phys, logi = _run_topk(csa, logits, [5000], pt)
    assert np.array_equal(logi[0], np.arange(512)) and np.array_equal(phys[0], np.arange(512))


# ------------------------------------------------------------------ attention


def _attn_case(g, fmt, B, Ls, H, ps_c=64, extra=3):
    """Pools with random page tables; raw pool shares the c4 page table."""
    pps = max((L + 255) // 256 for L in Ls)
    num_pages = B * pps + extra
    pt = gen.page_table(g, B, pps, num_pages)
    c4 = O.KVPool(*O.quant_kv_entries(gen.normal(g, (num_pages * ps_c, 576)), fmt), fmt)
    raw = O.KVPool(*O.quant_kv_entries(gen.normal(g, (num_pages * 256, 576)), fmt), fmt)
    return pt, c4, raw


@pytest.mark.parametrize("H,fmt,Ls,out_f32", [
    (64, "fp8", [131072 // 16, 700, 100, 2 * 4 + 1], False),  # full 512 + window, short, p < 127
    (128, "fp8", [20000, 3000], True),  # two-phase path (value copy), fp32 output
    # two-phase path with 16 queries: phase B gathers its values from the pools
    (64, "fp8", [131072 // 16 + 997 * i for i in range(14)] + [700, 9], True),
    (64, "fp8", [20 + 3 * i for i in range(130)], False),  # > 128 queries: split + combine path
    (32, "fp8", [20000, 131, 9, 3000], True),  # two 16-head pairs, fp32 output
    (16, "fp8", [5000, 700, 9], False),  # one 16-head pair
    (16, "f32", [4096, 333], True),
])
def test_csa_attention(csa, H, fmt, Ls, out_f32):
    g = gen.rng(1000 + H)
    B = len(Ls)
    pt, c4, raw = _attn_case(g, fmt, B, Ls, H)
    sel_phys = np.full((B, 512), -1, np.int32)
    for t, L in enumerate(Ls):
        n = L // 4
        logits = g.standard_normal(n)
        sel_phys[t] = O.topk_page_select(logits, n, pt[t])[0]
    qf = gen.normal(g, (B, H, 576))
    if fmt == "fp8":
        q, qh = _bf16(qf)
    else:
        q, qh = t_dev(qf), qf
    out = torch.empty((B, H, 512), dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    dc4, draw = kv_pool_to_device(c4, 64), kv_pool_to_device(raw, 256)
    scale = 576 ** -0.5
    csa.csa_sparse_attn(q, t_dev(np.arange(B, dtype=np.int32)), t_dev(np.array(Ls, np.int32) - 1),
                        t_dev(sel_phys), dc4, draw, t_dev(pt), 128, scale, out)
    got = out.float().cpu().numpy()
    for t, L in enumerate(Ls):
        p = L - 1
        sel = sel_phys[t][sel_phys[t] >= 0]
        win = O.page_slot(pt[t], O.window_positions(p, 128), 256)
        want = O.csa_attention_query(qh[t], c4.rows(sel), raw.rows(win), scale)
        if fmt == "f32":
            err = np.abs(got[t] - want).max(axis=1) / np.abs(want).max(axis=1)
            assert err.max() <= 1e-4, err.max()
        else:
            assert np.abs(got[t] - want).max() <= 2e-2


@pytest.mark.parametrize("fmt,Ls,H", [("fp8", [100, 128 * 40 + 77, 60000], 64),  # two-phase path
                                      ("fp8", [100, 128 * 40 + 77, 1048576 // 8], 64),
                                      ("fp8", [400000, 1000], 64),  # long list: many splits
                                      # 64 ragged lists (the most the length-balanced splits take)
                                      ("fp8", [int(500 * 1.085 ** i) for i in range(64)], 64),
                                      ("f32", [127, 128 * 9], 16)])
def test_hca_attention(csa, fmt, Ls, H):
    g = gen.rng(1100 + H)
    B = len(Ls)
    ratio = 128
    # HCA pool: its own page table with 64 entries per page
    hpp = max(L // ratio // 64 + 1 for L in Ls)
    hca_pages = B * hpp + 2
    hpt = gen.page_table(g, B, hpp, hca_pages)
    hca = O.KVPool(*O.quant_kv_entries(gen.normal(g, (hca_pages * 64, 576)), fmt), fmt)
    # raw pool: only the window's pages are read; every other page of the
    # table points at page 0, which holds values that must not matter
    rpp = max((L + 255) // 256 for L in Ls)
    rpt = np.zeros((B, rpp), np.int32)
    nxt = 1
    for t, L in enumerate(Ls):
        for pg in sorted(set(O.window_positions(L - 1, 128) // 256)):
            rpt[t, pg] = nxt
            nxt += 1
    raw = O.KVPool(*O.quant_kv_entries(gen.normal(g, (nxt * 256, 576)), fmt), fmt)
    qf = gen.normal(g, (B, H, 576))
    if fmt == "fp8":
        q, qh = _bf16(qf)
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    else:
        q, qh = t_dev(qf), qf
        out = torch.empty((B, H, 512), dtype=torch.float32, device=DEV)
    scale = 576 ** -0.5
    csa.hca_dense_attn(q, t_dev(np.arange(B, dtype=np.int32)), t_dev(np.array(Ls, np.int32) - 1),
                       max(Ls), ratio, kv_pool_to_device(hca, 64), t_dev(hpt),
                       kv_pool_to_device(raw, 256), t_dev(rpt), 128, scale, out)
    got = out.float().cpu().numpy()
    for t, L in enumerate(Ls):
        want = O.hca_query(hca, raw, hpt[t], rpt[t], L - 1, ratio, qh[t], 128, scale)
        if fmt == "f32":
            err = np.abs(got[t] - want).max(axis=1) / np.abs(want).max(axis=1)
            assert err.max() <= 1e-4, err.max()
        else:
            assert np.abs(got[t] - want).max() <= 2e-2


# ------------------------------------------------------------------ argument checks


def test_invalid_arguments_touch_nothing(csa):
    out = torch.full((2, 512), -5, dtype=torch.int32, device=DEV)
    logits = torch.zeros((2, 100), device=DEV)
    with pytest.raises(csa.CsaError) as e:
        csa.topk512_page_select(logits, torch.zeros(2, dtype=torch.int32, device=DEV),
                                torch.zeros(2, dtype=torch.int32, device=DEV),
                                torch.zeros((2, 1), dtype=torch.int32, device=DEV), out,
                                c4_page_size=0)
    assert e.value.status == csa.CSA_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.all(out == -5)


# ------------------------------------------------------------------ end to end


@pytest.mark.parametrize("seed_offset", [0, 1])
def test_tiny_fp32_decode_end_to_end(csa, seed_offset):
    from tests.e2e_tiny import run_tiny_decode_check
    res = run_tiny_decode_check(csa, torch, seed_offset)
    assert res["topk_equal"] or "attn_rel_err" not in res


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("lens", [
    [5000, 513, 64 * 7 + 3, 17, 0],     # fused: 512-entry scan chunks, ragged, an empty row
    [20000 - 37 * i for i in range(8)],  # fused: 1024-entry chunks
    [40000, 3000],                       # 79 chunks per row: merged into 8 lists first
])
def test_indexer_topk512(csa, fmt, lens):
    """indexer_topk512 against the oracle: each row's selection equals the top-512
    of the oracle's logits outside the near-tie band (entries within 1e-4 of the
    row's max |logit| of the 512-th largest), the physical slots are the page
    translation of the logical ones, and the result is bit for bit the one of
    indexer_score + topk512_page_select."""
    from tests.fullsize import topk_agrees
    g = gen.rng(1300 + len(fmt) + len(lens))
    T = len(lens)
    pt, pool, _ = _index_case(g, fmt, T, [max(n, 1) for n in lens])
    qraw = gen.normal(g, (T, 64, 128))
    qcodes, qsc = O.index_prep(qraw, True, fmt)
    w = gen.uniform(g, (T, 64))
    qfmt = csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_MXFP4
    qs = t_dev(qsc.astype(np.float32)) if fmt == "fp8" else t_dev(qsc)
    dpool = index_pool_to_device(pool, 64, 128)
    row_seq, row_len, dpt = t_dev(np.arange(T, dtype=np.int32)), t_dev(np.array(lens, np.int32)), t_dev(pt)
    maxn = max(lens)
    phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(t_dev(qcodes), t_dev(w), row_seq, row_len, maxn, dpt, dpool, phys, logi,
                        q_fmt=qfmt, q_scale=qs)
    # the two calls
    logits = torch.empty((T, maxn), device=DEV)
    csa.indexer_score(t_dev(qcodes), t_dev(w), row_seq, row_len, maxn, dpt, dpool, logits,
                      q_fmt=qfmt, q_scale=qs)
    phys2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    logi2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    csa.topk512_page_select(logits, row_len, row_seq, dpt, phys2, logi2)
    gp, gl = phys.cpu().numpy(), logi.cpu().numpy()
    assert np.array_equal(gp, phys2.cpu().numpy()) and np.array_equal(gl, logi2.cpu().numpy())
    qhat = O.index_dequant(qcodes, qsc, fmt)
    for t, n in enumerate(lens):
        k = min(512, n)
        assert np.all(gl[t, k:] == -1) and np.all(gp[t, k:] == -1), f"row {t}: tail not -1"
        if n == 0:
            continue
        assert np.all(np.diff(gl[t, :k]) > 0), f"row {t}: not ascending"
        assert np.array_equal(gp[t, :k], O.page_slot(pt[t], gl[t, :k], 64)), f"row {t}: slots"
        want = O.indexer_logits(qhat[t], w[t], pool.rows(O.page_slot(pt[t], np.arange(n), 64)))
        ok, _, nband = topk_agrees(want, gl[t], 512, 1e-4 * np.abs(want).max())
        assert ok, f"row {t}: selection differs outside the near-tie band ({nband} in band)"


def test_indexer_topk512_f32_two_calls(csa):
    """An fp32 index pool takes the two-call path (logits in the workspace):
    the selection is the top-512 of the oracle's logits outside the near-tie
    band, and equal to indexer_score + topk512_page_select."""
    from tests.fullsize import topk_agrees
    g = gen.rng(1350)
    lens = [3000, 700, 5]
    T = len(lens)
    pt, pool, _ = _index_case(g, "f32", T, lens, H=8, D=64)
    q = gen.normal(g, (T, 8, 64))
    w = gen.uniform(g, (T, 8))
    dpool = index_pool_to_device(pool, 64, 64)
    row_seq, row_len, dpt = t_dev(np.arange(T, dtype=np.int32)), t_dev(np.array(lens, np.int32)), t_dev(pt)
    phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(t_dev(q), t_dev(w), row_seq, row_len, max(lens), dpt, dpool, phys, logi)
    logits = torch.empty((T, max(lens)), device=DEV)
    csa.indexer_score(t_dev(q), t_dev(w), row_seq, row_len, max(lens), dpt, dpool, logits)
    logi2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    phys2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    csa.topk512_page_select(logits, row_len, row_seq, dpt, phys2, logi2)
    gl = logi.cpu().numpy()
    assert np.array_equal(gl, logi2.cpu().numpy()) and np.array_equal(phys.cpu().numpy(), phys2.cpu().numpy())
    for t, n in enumerate(lens):
        want = O.indexer_logits(q[t], w[t], pool.rows(O.page_slot(pt[t], np.arange(n), 64)))
        ok, _, nband = topk_agrees(want, gl[t], 512, 1e-4 * np.abs(want).max())
        assert ok, f"row {t}: selection differs outside the near-tie band ({nband} in band)"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_indexer_many_rows_causal(csa, fmt):
    """Prefill shape: hundreds of query rows of one sequence with the causal
    row length min(N, (p+1)/4), plus a block of rows from a second sequence
    (read from its own pages) and a group whose first rows are empty; every
    row within 1e-4 of its max."""
    g = gen.rng(1200 + len(fmt))
    L1, L2 = 21000, 9000
    N1, N2 = L1 // 4, L2 // 4
    pt, pool, _ = _index_case(g, fmt, 2, [N1, N2])
    T = 300
    pos = np.arange(L1 - T, L1)
    row_seq = np.zeros(T, np.int32)
    row_len = np.minimum(N1, (pos + 1) // 4).astype(np.int32)
    row_seq[100:108] = 1
    row_len[100:108] = N2 - np.arange(8)
    # a group of rows whose first sequence has nothing to score: the other
    # sequence's rows still run
    row_len[200:204] = 0
    row_seq[204:208] = 1
    row_len[204:208] = N2 // 2 + np.arange(4)
    qraw = gen.normal(g, (T, 64, 128))
    qcodes, qsc = O.index_prep(qraw, True, fmt)
    w = gen.uniform(g, (T, 64))
    logits = torch.full((T, N1), float("nan"), device=DEV)
    qfmt = csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_MXFP4
    qs = t_dev(qsc.astype(np.float32)) if fmt == "fp8" else t_dev(qsc)
    csa.indexer_score(t_dev(qcodes), t_dev(w), t_dev(row_seq), t_dev(row_len), N1, t_dev(pt),
                      index_pool_to_device(pool, 64, 128), logits, q_fmt=qfmt, q_scale=qs)
    got = logits.cpu().numpy()
    qhat = O.index_dequant(qcodes, qsc, fmt)
    for t in list(range(0, 12)) + list(range(96, 112)) + list(range(198, 210)) + list(range(T - 12, T)):
        n = int(row_len[t])
        if n == 0:
            assert np.all(np.isnan(got[t])), f"row {t} has no entries but was written"
            continue
        want = O.indexer_logits(qhat[t], w[t], pool.rows(O.page_slot(pt[row_seq[t]], np.arange(n), 64)))
        np.testing.assert_allclose(got[t, :n], want, rtol=0, atol=1e-4 * np.abs(want).max())
        assert np.all(np.isnan(got[t, n:])), f"row {t} wrote past row_len"


@pytest.mark.parametrize("fmt,q_len", [("fp8", 4), ("mxfp4", 8), ("fp8", 2), ("fp8", 6), ("fp8", 5),
                                       ("mxfp4", 3), ("fp8", 10)])
def test_indexer_rows_per_seq(csa, fmt, q_len):
    """Multi-token decode: q_len query rows per sequence (positions L-q_len ..
    L-1, causal row length min(N, (p+1)/4)) with the CSA_ROWS_PER_SEQ hint,
    which sends each group's rows to the row-block kernel over page ranges.
    Every row within 1e-4 of its max of the oracle's logits; rows past their
    row_len untouched; a row whose sequence differs from its group's (the hint
    broken on purpose) still scored from its own pages; indexer_topk512 with
    the hint equal to indexer_score + topk512_page_select."""
    g = gen.rng(1250 + q_len + len(fmt))
    lens = [131072 // 8 + 4 * 997 + 3, 20000, 4096 + 1, 900]  # raw lengths
    S = len(lens)
    Ns = [L // 4 for L in lens]
    pt, pool, _ = _index_case(g, fmt, S, Ns)
    T = S * q_len
    row_seq = np.repeat(np.arange(S, dtype=np.int32), q_len)
    pos = np.concatenate([np.arange(L - q_len, L) for L in lens])
    row_len = np.minimum(np.repeat(Ns, q_len), (pos + 1) // 4).astype(np.int32)
    row_seq[q_len + 1] = 3  # breaks the hint: read from its own pages
    row_len[q_len + 1] = Ns[3]
    qraw = gen.normal(g, (T, 64, 128))
    qcodes, qsc = O.index_prep(qraw, True, fmt)
    w = gen.uniform(g, (T, 64))
    maxn = max(Ns)
    qfmt = csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_MXFP4
    qs = t_dev(qsc.astype(np.float32)) if fmt == "fp8" else t_dev(qsc)
    dpool = index_pool_to_device(pool, 64, 128)
    hint = csa.CSA_ROWS_PER_SEQ(q_len)
    drs, drl, dpt = t_dev(row_seq), t_dev(row_len), t_dev(pt)
    logits = torch.full((T, maxn), float("nan"), device=DEV)
    csa.indexer_score(t_dev(qcodes), t_dev(w), drs, drl, maxn, dpt, dpool, logits, q_fmt=qfmt,
                      q_scale=qs, prep=hint)
    got = logits.cpu().numpy()
    qhat = O.index_dequant(qcodes, qsc, fmt)
    for t in range(T):
        n = int(row_len[t])
        want = O.indexer_logits(qhat[t], w[t], pool.rows(O.page_slot(pt[row_seq[t]], np.arange(n), 64)))
        np.testing.assert_allclose(got[t, :n], want, rtol=0, atol=1e-4 * np.abs(want).max(),
                                   err_msg=f"row {t}")
        assert np.all(np.isnan(got[t, n:])), f"row {t} wrote past row_len"
    phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(t_dev(qcodes), t_dev(w), drs, drl, maxn, dpt, dpool, phys, logi, q_fmt=qfmt,
                        q_scale=qs, prep=hint)
    phys2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    logi2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    csa.topk512_page_select(logits.nan_to_num(nan=-float("inf")), drl, drs, dpt, phys2, logi2)
    assert np.array_equal(phys.cpu().numpy(), phys2.cpu().numpy())
    assert np.array_equal(logi.cpu().numpy(), logi2.cpu().numpy())


# ------------------------------------------------------------------ fused decode preparation


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_decode_prep(csa, fmt):
    """csa_decode_prep against the oracle: the block a token completes (and only
    then) is compressed into the C4 pool and its index-K row prepared into the
    index pool; the token is stored in the raw pool; the query rows are
    prepared. Sequences whose token completes no block (L % 4 != 0, or p < 3)
    leave both pools untouched."""
    g = gen.rng(1300 + len(fmt))
    lens = np.array([4096, 4099, 12, 3, 8192 + 256, 5], np.int64)
    B, ratio, H_I = len(lens), 4, 64
    pos = (lens - 1).astype(np.int32)
    pps = int(max((L + 255) // 256 for L in lens))
    P = B * pps + 3
    pt = gen.page_table(g, B, pps, P)
    w, b = gen.gate_params(g, ratio)
    x, xh = _bf16(gen.normal(g, (B, ratio, 576)))
    k, kh = _bf16(gen.normal(g, (B, 128)))
    q, qh = _bf16(gen.normal(g, (B, H_I, 128)))
    kfmt = csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_MXFP4
    c4 = csa.alloc_kv_pool(P, 64, csa.CSA_FP8_E4M3)
    raw = csa.alloc_kv_pool(P, 256, csa.CSA_FP8_E4M3)
    kpool = csa.alloc_index_pool(P, 64, 128, kfmt)
    if fmt == "fp8":
        q_out = torch.empty((B, H_I, 128), dtype=torch.uint8, device=DEV)
        q_sc = torch.empty((B, H_I), dtype=torch.float32, device=DEV)
    else:
        q_out = torch.empty((B, H_I, 64), dtype=torch.uint8, device=DEV)
        q_sc = torch.empty((B, H_I, 4), dtype=torch.uint8, device=DEV)
    csa.csa_decode_prep(x, t_dev(pos), t_dev(w), t_dev(b), t_dev(pt), c4, t_dev(pt), raw,
                        k_rows=k, q_rows=q, kpool=kpool, q_out=q_out, q_out_scale=q_sc)
    torch.cuda.synchronize()
    lat = c4.latent.cpu().numpy().reshape(-1, 512)
    sc = c4.scale.cpu().numpy().reshape(-1)
    rope = c4.rope.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1, 64)
    kd = kpool.data.cpu().numpy().reshape(P * 64, -1)
    ks = kpool.scale.cpu().numpy().reshape(P * 64, -1)
    written = np.zeros(P * 64, bool)
    for s in range(B):
        L = int(lens[s])
        if L % ratio or L < ratio:
            continue
        kb = L // ratio - 1
        slot = int(O.page_slot(pt[s], kb, 64))
        written[slot] = True
        c = O.compress_blocks(xh[s], L - ratio, ratio, w, b)
        oc, osc, orope = O.quant_kv_entries(c, "fp8")
        np.testing.assert_allclose(sc[slot], osc[0], rtol=3e-6)
        ok, _ = fp8_codes_match(lat[slot][None], oc, c[:, :512].astype(np.float32) / osc[:, None],
                                rel=2e-5)
        assert ok, f"sequence {s}: compressed latent differs"
        gr, orr = O.bf16_decode(rope[slot]), O.bf16_decode(orope[0])
        assert np.all(np.abs(gr - orr) <= 2.0 ** -7 * np.abs(orr) + 1e-5)
        codes, scale = O.index_prep(kh[s:s + 1], True, fmt)
        assert np.array_equal(kd[slot], codes[0].reshape(-1)), f"sequence {s}: index-K row differs"
        assert np.array_equal(ks[slot].view(np.uint8), np.asarray(scale[0]).reshape(-1).view(np.uint8))
    # nothing else of either pool was written (poison bytes 0xFF remain)
    assert np.all(lat[~written] == 0xFF) and np.all(kd[~written] == 0xFF)
    # the token of every sequence, in the raw pool
    rl = raw.latent.cpu().numpy().reshape(-1, 512)
    rs = raw.scale.cpu().numpy().reshape(-1)
    rr = raw.rope.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1, 64)
    for s in range(B):
        p = int(pos[s])
        slot = int(O.page_slot(pt[s], p, 256))
        oc, osc, orope = O.quant_kv_entries(xh[s, ratio - 1:ratio], "fp8")
        assert rs[slot] == np.float32(osc[0])
        assert np.array_equal(rl[slot], oc[0]) and np.array_equal(rr[slot], orope[0])
    # the prepared query rows
    codes, scale = O.index_prep(qh.reshape(-1, 128), True, fmt)
    assert np.array_equal(q_out.cpu().numpy().reshape(B * H_I, -1), codes.reshape(B * H_I, -1))
    assert np.array_equal(q_sc.cpu().numpy().reshape(B * H_I, -1).view(np.uint8),
                          np.asarray(scale).reshape(B * H_I, -1).view(np.uint8))
