"""GPU parity: each entry point of libcsa.so against the CPU oracle on the same
seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles / pages and a ragged tail.

Bars: index and selection work bit-exact; quantised codes equal except a
one-code step where the oracle's exact (float64) pre-rounding value lies
within the float32 evaluation error bound of a rounding midpoint
(tests/quant_band.py states the bounds); logits within 1e-4 of the row's max
magnitude, widened only by what such in-band codes can change; attention
within 1e-4 (relative to the row's max) for the fp32 path and 2e-2 max-abs for
the bf16 / FP8 path.
"""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests import quant_band as Q
from tests.gpu_helpers import (DEV, index_pool_to_device, kv_pool_to_device, t_dev)
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
    ok, msg, _ = Q.fp8_rows_match(out.cpu().numpy(), sc.cpu().numpy(), Q.exact_rotated(vh, True),
                                  Q.rotation_error_bound(vh, 128))
    assert ok, msg


@pytest.mark.parametrize("rows", [5, 1000])
def test_index_prep_mxfp4_hadamard(csa, rows):
    g = gen.rng(200 + rows)
    v, vh = _bf16(gen.normal(g, (rows, 128)))
    out = torch.empty((rows, 64), dtype=torch.uint8, device=DEV)
    sc = torch.empty((rows, 4), dtype=torch.uint8, device=DEV)
    csa.csa_index_prep(v, 128, csa.CSA_PREP_HADAMARD, csa.CSA_MXFP4, out, sc)
    ok, msg, _ = Q.mxfp4_rows_match(out.cpu().numpy(), sc.cpu().numpy(), Q.exact_rotated(vh, True),
                                    Q.rotation_error_bound(vh, 128))
    assert ok, msg


def _rope_table(max_pos, rope_dim):
    """The caller's cos/sin table (float32 [max_pos, rope_dim/2, 2]) of the
    textbook RoPE angles, from the oracle's definition."""
    cos, sin = O.rope_cos_sin(np.arange(max_pos), rope_dim)
    return np.stack([cos, sin], axis=-1).astype(np.float32)


@pytest.mark.parametrize("fmt,hadamard", [("fp8", True), ("mxfp4", True), ("f32", True),
                                          ("f32", False)])
def test_index_prep_rope(csa, fmt, hadamard):
    """rope -> hadamard -> quant of query-shaped rows [T][64][128] (64 rows per
    position) against the oracle's exact rotation of the same rows with the
    same table values, within the float32 evaluation band."""
    g = gen.rng(150 + len(fmt) + hadamard)
    T, H, D, rd = 7, 64, 128, 64
    pos = np.array([0, 1, 5, 4095, 65536, 131071, 140000 - 1], np.int32)
    table = _rope_table(140000, rd)
    v, vh = _bf16(gen.normal(g, (T * H, D)))
    out = torch.full((T * H, D // 2 if fmt == "mxfp4" else D), 0xAB, dtype=torch.uint8, device=DEV)
    if fmt == "f32":
        out = torch.full((T * H, D), float("nan"), dtype=torch.float32, device=DEV)
        sc = None
    elif fmt == "fp8":
        sc = torch.empty(T * H, dtype=torch.float32, device=DEV)
    else:
        sc = torch.empty((T * H, D // 32), dtype=torch.uint8, device=DEV)
    flags = csa.CSA_PREP_ROPE | (csa.CSA_PREP_HADAMARD if hadamard else 0)
    ofmt = {"fp8": csa.CSA_FP8_E4M3, "mxfp4": csa.CSA_MXFP4, "f32": csa.CSA_F32}[fmt]
    csa.csa_index_prep(v, D, flags, ofmt, out, sc, rope_pos=t_dev(pos), rope_table=t_dev(table),
                       rows_per_pos=H)
    cs = table[np.repeat(pos, H)].astype(np.float64)
    rope = (cs[..., 0], cs[..., 1], rd)
    exact = Q.exact_rotated(vh, hadamard, rope=rope)
    err = Q.rotation_error_bound(vh, D, rope=True) if hadamard else 2.0 ** -22 * np.abs(vh).sum(axis=1)
    if fmt == "fp8":
        ok, msg, _ = Q.fp8_rows_match(out.cpu().numpy(), sc.cpu().numpy(), exact, err)
    elif fmt == "mxfp4":
        ok, msg, _ = Q.mxfp4_rows_match(out.cpu().numpy(), sc.cpu().numpy(), exact, err)
    else:
        got = out.cpu().numpy()
        ok = bool(np.all(np.abs(got - exact) <= err[:, None] + 2.0 ** -24 * np.abs(exact)))
        msg = f"max deviation {np.abs(got - exact).max()}"
        # the first D - rope_dim dims of an unrotated row are untouched
        if not hadamard:
            ok = ok and np.array_equal(got[:, :D - rd], vh[:, :D - rd])
    assert ok, msg


def test_index_prep_f32_dst_rows(csa):
    """Rows go to dst_rows[i]; a negative destination skips the row."""
    g = gen.rng(300)
    v = gen.normal(g, (50, 64))
    dst = np.random.default_rng(1).permutation(80)[:50].astype(np.int32)
    dst[[3, 17, 49]] = -1
    out = torch.full((80, 64), float("nan"), dtype=torch.float32, device=DEV)
    csa.csa_index_prep(t_dev(v), 64, csa.CSA_PREP_HADAMARD, csa.CSA_F32, out, None, t_dev(dst))
    want = O.hadamard_rotate(v)
    err = Q.rotation_error_bound(v, 64)
    got = out.cpu().numpy()
    keep = dst >= 0
    assert np.all(np.abs(got[dst[keep]] - want[keep]) <= err[keep, None])
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
    for s in range(2):
        xs = xh[cu[s]:cu[s + 1]]
        c = O.compress_blocks(xs, starts[s], ratio, w, b)
        kb0 = starts[s] // ratio
        slots = O.page_slot(pt[s], np.arange(kb0, kb0 + len(c)), 64)
        # every block's evaluation error bound (float32 gates and pooling)
        first = (-starts[s]) % ratio  # rows before the first aligned block
        err = np.stack([Q.compress_error_bound(xs[first + k * ratio:first + (k + 1) * ratio], w)
                        for k in range(len(c))])
        # FP8 latent: scale and codes within the band of the exact pooled value
        ok, msg, _ = Q.fp8_rows_match(lat[slots], sc[slots], c[:, :512], err[:, :512])
        assert ok, msg
        # bf16 RoPE dims: one ulp only where the exact value is within the band of the midpoint
        ok, msg = Q.bf16_match(rope[slots], c[:, 512:], err[:, 512:])
        assert ok, msg


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
    qe, qerr = Q.exact_rotated(qh, True), Q.rotation_error_bound(qh, 128)
    match = Q.fp8_rows_match if fmt == "fp8" else Q.mxfp4_rows_match
    ok, msg, _ = match(qu.cpu().numpy(), qus.cpu().numpy(), qe, qerr)
    assert ok, msg
    dq = Q.band_delta(qe, qerr, fmt)
    qhat = O.index_dequant(qcodes, qsc, fmt)
    got = logits.cpu().numpy()
    for t, n in enumerate(lens):
        khat = pool.rows(O.page_slot(pt[t], np.arange(n), 64))
        want = O.indexer_logits(qhat[t], w[t], khat)
        slack = Q.logit_slack(qhat[t], dq[t], w[t], khat, np.zeros_like(khat))
        assert np.all(np.abs(got[t, :n] - want) <= 1e-4 * np.abs(want).max() + slack)


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
    # 70 queries x 2 head blocks: two uniform splits + combine, fp32 output
    (128, "fp8", [2050 + 3 * i for i in range(69)] + [9], True),
    # 32 and 31 queries: more 64-entry chunks than CUs, so 96-entry chunks
    # (the last one partly past the list)
    (64, "fp8", [131072 // 16 + 997 * i for i in range(28)] + [700, 100, 9, 5000], False),
    (64, "fp8", [20000 + 4099 * i for i in range(29)] + [130, 9], True),
    # 48 queries: more workgroups than CUs even with 96-entry chunks, so
    # 64-entry chunks, two workgroups per CU
    (64, "fp8", [9000 + 131 * i for i in range(47)] + [77], True),
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
                                      # 32 lists of up to 748 entries: 96-entry chunks
                                      ("fp8", [int(2000 * 1.126 ** i) for i in range(32)], 64),
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
    assert res["attn_rel_err"] <= 1e-4


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("lens", [
    [5000, 513, 64 * 7 + 3, 17, 0],     # fused: 512-entry scan chunks, ragged, an empty row
    [20000 - 37 * i for i in range(8)],  # fused: 1024-entry chunks
    [40000, 3000],                       # 79 chunks per row: merged into 8 lists first
    [60000] + [1000 + 37 * i for i in range(19)],  # ragged: 300 chunk workgroups (two rounds)
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


_LONG_POOLS = {}


def _long_pool(fmt, pages):
    """A pool of `pages` 64-entry pages of prepared index-K rows, drawn once per format."""
    if (fmt, pages) not in _LONG_POOLS:
        g = gen.rng(1390 + len(fmt))
        data, sc = O.index_prep(gen.normal(g, (pages * 64, 128)), True, fmt)
        _LONG_POOLS[(fmt, pages)] = O.IndexPool(data, sc, fmt)
    return _LONG_POOLS[(fmt, pages)]


def _long_chunk(lens, slots=256):
    """The scan chunk length the library takes for a batch with more live
    4096-entry chunks than workgroups resident at once: of 4096, 4608 and
    5120 entries, the fewest entries per workgroup slot over the rounds."""
    best = None
    for c in (4096, 4608, 5120):
        live = sum((n + c - 1) // c for n in lens)
        cost = -(-live // slots) * c
        if best is None or cost < best[0]:
            best = (cost, c)
    return best[1]


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("case", ["ragged16_c5120", "rows30_c4608", "rows40_final_c4608",
                                  "rows100_final_c5120", "rows70_c4096", "rows70_empty_short",
                                  "rows100_final_empty_short"])
def test_indexer_topk512_long_batches(csa, fmt, case):
    """Batches with more live 4096-entry scan chunks than the GPU holds at
    once take longer chunks, chosen from the rows' lengths: 16 ragged rows of
    3K-234K entries (5120-entry chunks, finished inside the scan in up to 6
    groups), 30 rows of ~36000 (4608, finished inside the scan), 40 rows of
    ~27000 (4608, through the final pass, a chunk of padding per row), and
    with more than 64 rows (the plan over four 64-row blocks per lane) 100
    rows of ~10000 (5120, final pass) and 70 rows of ~40000 (4096 in three
    rounds, finished inside the scan); both last ones again with empty rows
    and rows shorter than 512. Bit for bit the two-call path; sampled rows
    (the longest, a middle one, the shortest non-empty one) against the
    oracle's top-512."""
    from tests.fullsize import topk_agrees
    if case == "ragged16_c5120":
        lens = [int(n) for n in gen.ragged_lengths(gen.rng(1005), 16, 8192, 1 << 20) // 4]
        want_chunk = 5120
    elif case == "rows30_c4608":
        lens = [36000 - 3 * i for i in range(30)]
        want_chunk = 4608
    elif case == "rows40_final_c4608":
        lens = [27000 - 5 * i for i in range(40)]
        want_chunk = 4608
    elif case.startswith("rows100_final"):
        lens = [10000 - 3 * i for i in range(100)]
        want_chunk = 5120
    else:
        lens = [40000 - 7 * i for i in range(70)]
        want_chunk = 4096
    if case.endswith("empty_short"):
        for i in (0, 5, 17, len(lens) - 1):
            lens[i] = 0
        for i in (6, 41):
            lens[i] = 300 + i
    assert sum((n + 4095) // 4096 for n in lens) > 256 and _long_chunk(lens) == want_chunk
    g = gen.rng(1380 + len(fmt) + len(case))
    T = len(lens)
    # one pool of 4096 pages; each row's page table a prefix of its own
    # permutation (no page twice in a row; rows share pages)
    pool_pages = 4096
    pps = max((n + 63) // 64 for n in lens)
    pt = np.stack([g.permutation(pool_pages)[:pps] for _ in lens]).astype(np.int32)
    pool = _long_pool(fmt, pool_pages)
    qcodes, qsc = O.index_prep(gen.normal(g, (T, 64, 128)), True, fmt)
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
        if n == 0:
            assert np.all(gl[t] == -1) and np.all(gp[t] == -1), f"row {t}: empty row not -1"
    order = [t for t in np.argsort(lens) if lens[t] > 0]
    for t in (int(order[-1]), int(order[len(order) // 2]), int(order[0])):
        n = lens[t]
        k = min(512, n)
        assert np.all(gl[t, k:] == -1) and np.all(gp[t, k:] == -1), f"row {t}: tail not -1"
        assert np.all(np.diff(gl[t, :k]) > 0), f"row {t}: not ascending"
        assert np.array_equal(gp[t, :k], O.page_slot(pt[t], gl[t, :k], 64)), f"row {t}: slots"
        want = O.indexer_logits(qhat[t], w[t], pool.rows(O.page_slot(pt[t], np.arange(n), 64)))
        ok, _, nband = topk_agrees(want, gl[t], 512, 1e-4 * np.abs(want).max())
        assert ok, f"row {t}: selection differs outside the near-tie band ({nband} in band)"


def test_indexer_topk512_side_stream(csa):
    """A call enqueued on a stream other than the current one, with the
    library's temporary workspace: it is allocated and zero-filled on that
    stream (the in-scan finish counts arrivals in it), and the selection is
    bit for bit the one made on the current stream."""
    g = gen.rng(1395)
    lens = [20000 - 37 * i for i in range(8)]  # 20 chunks per row: finished inside the scan
    T = len(lens)
    pt, pool, _ = _index_case(g, "fp8", T, lens)
    qcodes, qsc = O.index_prep(gen.normal(g, (T, 64, 128)), True, "fp8")
    w = gen.uniform(g, (T, 64))
    dpool = index_pool_to_device(pool, 64, 128)
    args = (t_dev(qcodes), t_dev(w), t_dev(np.arange(T, dtype=np.int32)),
            t_dev(np.array(lens, np.int32)), max(lens), t_dev(pt), dpool)
    qs = t_dev(qsc.astype(np.float32))
    p1 = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(*args, p1, q_fmt=csa.CSA_FP8_E4M3, q_scale=qs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    p2 = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    for _ in range(3):  # repeated: each call's counters must start at zero
        csa.indexer_topk512(*args, p2, q_fmt=csa.CSA_FP8_E4M3, q_scale=qs, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)


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


@pytest.mark.parametrize("fmt,case", [("fp8", "ranges"), ("mxfp4", "ranges"), ("fp8", "direct"),
                                      ("mxfp4", "direct"), ("fp8", "ties_direct"),
                                      ("fp8", "ties_ranges")])
def test_indexer_topk512_many_rows(csa, fmt, case):
    """Prefill shape through indexer_topk512: the row-block kernel keeps each
    row's top-512 as it scores (no logits written). With one page range per
    row it writes the selection itself ("direct"), with several a final pass
    merges the ranges' candidates ("ranges"). Bit for bit the result of
    indexer_score + topk512_page_select, including rows of another sequence
    than their group's first row, empty rows, rows shorter than 512, and index
    pools whose rows repeat (many exactly equal logits: equal keys go to the
    lower index)."""
    g = gen.rng(1400 + len(fmt) + len(case))
    ties = case.startswith("ties")
    if case.endswith("ranges"):
        L1, L2, T = 21000, 9000, 300   # 83 pages: 10 ranges of 9 pages
    else:
        L1, L2, T = 3600, 2000, 520    # 15 pages: one range
    N1, N2 = L1 // 4, L2 // 4
    pt, pool, num_pages = _index_case(g, fmt, 2, [N1, N2])
    if ties:  # index-K rows repeat with period 7: logits repeat exactly
        rows = np.arange(num_pages * 64) % 7
        pool = O.IndexPool(pool.data[rows], pool.scale[rows], fmt)
    pos = np.arange(L1 - T, L1)
    row_seq = np.zeros(T, np.int32)
    row_len = np.minimum(N1, (pos + 1) // 4).astype(np.int32)
    row_len[:8] = [0, 1, 63, 64, 65, 511, 512, 513]
    row_seq[100:108] = 1
    row_len[100:108] = N2 - np.arange(8)
    row_len[200:204] = 0
    row_seq[204:208] = 1
    row_len[204:208] = N2 // 2 + np.arange(4)
    qraw = gen.normal(g, (T, 64, 128))
    qcodes, qsc = O.index_prep(qraw, True, fmt)
    w = gen.uniform(g, (T, 64))
    qfmt = csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_MXFP4
    qs = t_dev(qsc.astype(np.float32)) if fmt == "fp8" else t_dev(qsc)
    dpool = index_pool_to_device(pool, 64, 128)
    drs, drl, dpt = t_dev(row_seq), t_dev(row_len), t_dev(pt)
    phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(t_dev(qcodes), t_dev(w), drs, drl, N1, dpt, dpool, phys, logi, q_fmt=qfmt,
                        q_scale=qs)
    logits = torch.full((T, N1), float("nan"), device=DEV)
    csa.indexer_score(t_dev(qcodes), t_dev(w), drs, drl, N1, dpt, dpool, logits, q_fmt=qfmt,
                      q_scale=qs)
    phys2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    logi2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    csa.topk512_page_select(logits, drl, drs, dpt, phys2, logi2)
    gp, gl = phys.cpu().numpy(), logi.cpu().numpy()
    wp, wl = phys2.cpu().numpy(), logi2.cpu().numpy()
    bad = [t for t in range(T) if not (np.array_equal(gl[t], wl[t]) and np.array_equal(gp[t], wp[t]))]
    assert not bad, f"{len(bad)} rows differ from the two calls, first {bad[:5]}"
    if ties:  # the case has many equal logits to break
        lg = logits.cpu().numpy()
        t = T - 1
        kth = np.sort(lg[t, :row_len[t]])[-512]
        assert np.sum(lg[t, :row_len[t]] == kth) > 1


@pytest.mark.parametrize("per_seq", [0, 4])
@pytest.mark.parametrize("case", ["rising", "special"])
def test_indexer_topk512_many_rows_adversarial(csa, case, per_seq):
    """The row-block kernel's running top-512 on the inputs that are hardest
    for it, bit for bit against indexer_score + topk512_page_select, with 8
    rows per workgroup (a wave per row) and, with the rows-per-sequence hint
    4, with 4 rows per workgroup (two waves per row, lists merged):
    "rising": every index-K row holds the same FP8 codes with a scale that
    grows with the entry, so each row's logits rise with j and every page's
    entries pass the threshold (a compaction every few pages);
    "special": head weights with NaN, +-inf, -0 and negative values in some
    rows, giving NaN, infinite and signed-zero logits (NaN ranks lowest, -0
    equals +0)."""
    g = gen.rng(1450 + len(case))
    L1, T = 12000, 264            # 3000 entries per row at most, 47 pages, 5 ranges
    N1 = L1 // 4
    pt, pool, num_pages = _index_case(g, "fp8", 1, [N1])
    if case == "rising":
        data = np.broadcast_to(pool.data[:1], pool.data.shape).copy()
        # entry j's scale grows with its logical index j: slot -> j through the table
        slot_j = np.zeros(num_pages * 64, np.int64)
        pages = pt[0]
        for j in range(N1):
            slot_j[pages[j // 64] * 64 + j % 64] = j
        scale = (pool.scale[0] * (1.0 + slot_j / N1)).astype(np.float32)
        pool = O.IndexPool(data, scale, "fp8")
    pos = np.arange(L1 - T, L1)
    row_seq = np.zeros(T, np.int32)
    row_len = np.minimum(N1, (pos + 1) // 4).astype(np.int32)
    qraw = gen.normal(g, (T, 64, 128))
    if case == "rising":
        # q sign-aligned with the shared K codes (no rotation of q, so that
        # every head's dot product is positive)
        qraw = np.abs(qraw) * np.sign(pool.data[0].view(np.int8).astype(np.float64) + 0.5)[None, None, :]
    qcodes, qsc = O.index_prep(qraw, case != "rising", "fp8")
    w = gen.uniform(g, (T, 64)).astype(np.float32)
    if case == "special":
        w[3, :] = np.nan                     # every logit NaN
        w[5, 7] = np.inf                     # +inf or NaN logits
        w[6, :] = -0.0                       # all logits zero (+0 or -0)
        w[7, :] = -w[7, :]                   # all logits <= 0
        w[9, 11] = -np.inf
    dpool = index_pool_to_device(pool, 64, 128)
    drs, drl, dpt = t_dev(row_seq), t_dev(row_len), t_dev(pt)
    qs = t_dev(qsc.astype(np.float32))
    hint = csa.CSA_ROWS_PER_SEQ(per_seq) if per_seq else 0
    phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(t_dev(qcodes), t_dev(w), drs, drl, N1, dpt, dpool, phys, logi,
                        q_fmt=csa.CSA_FP8_E4M3, q_scale=qs, prep=hint)
    logits = torch.full((T, N1), float("nan"), device=DEV)
    csa.indexer_score(t_dev(qcodes), t_dev(w), drs, drl, N1, dpt, dpool, logits,
                      q_fmt=csa.CSA_FP8_E4M3, q_scale=qs, prep=hint)
    phys2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    logi2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    csa.topk512_page_select(logits, drl, drs, dpt, phys2, logi2)
    gl, wl = logi.cpu().numpy(), logi2.cpu().numpy()
    bad = [t for t in range(T) if not np.array_equal(gl[t], wl[t])]
    assert not bad, f"{len(bad)} rows differ from the two calls, first {bad[:5]}"
    assert np.array_equal(phys.cpu().numpy(), phys2.cpu().numpy())
    lg = logits.cpu().numpy()
    if case == "rising":  # the logits do rise with j: the selection is each row's last 512
        t = T - 1
        n = row_len[t]
        assert np.all(np.diff(lg[t, :n]) >= 0)
        assert np.array_equal(gl[t], np.arange(n - 512, n))
    else:
        assert np.isnan(lg[3, :row_len[3]]).all()
        assert np.array_equal(gl[3], np.arange(512))  # all NaN: the lowest indices


@pytest.mark.parametrize("shape", ["wide", "long", "wide40"])
@pytest.mark.parametrize("case", ["ties", "outliers", "special"])
def test_indexer_topk512_decode_adversarial(csa, case, shape):
    """The decode scan's selection on inputs that defeat its shortcuts, bit
    for bit against indexer_score + topk512_page_select. Shapes: "wide", 32
    rows of ~32K entries (4096-entry chunks, 8 per row, a final pass);
    "long", 4 rows of ~131K (2048-entry chunks, 64 per row, finished inside
    the scan); "wide40", 40 rows of ~32K (320 chunk workgroups, more than
    CUs). Cases:
    "ties": index-K rows drawn from six distinct rows, so a row's logits take
    six values (every candidate reaches the bound); "outliers": a few entries
    with scales 1000x the rest, so the key range is wide and the threshold's
    bucket crowded; "special": head weights with NaN, +-inf, -0 and negative
    values (NaN logits rank lowest, -0 equals +0)."""
    g = gen.rng(1470 + len(case) + 10 * len(shape))
    if shape in ("wide", "wide40"):
        T, pps = (32 if shape == "wide" else 40), 512
        lens = [32768 - 997 * (t % 5) for t in range(T)]
    else:
        T, pps = 4, 2048
        lens = [131072, 131072 - 700, 131072 - 2048 * 9 - 5, 70000]
    num_pages = T * pps + 3
    pt = gen.page_table(g, T, pps, num_pages)
    distinct = 6 if case == "ties" else 4096
    kraw = gen.normal(g, (distinct, 128))
    d0, s0 = O.index_prep(kraw, True, "fp8")
    pick = g.integers(0, distinct, num_pages * 64)
    data, scale = d0[pick], s0[pick].astype(np.float32)
    if case == "outliers":
        scale[g.integers(0, num_pages * 64, 40)] *= 1000.0
    pool = O.IndexPool(data, scale, "fp8")
    qraw = gen.normal(g, (T, 64, 128))
    qcodes, qsc = O.index_prep(qraw, True, "fp8")
    w = gen.uniform(g, (T, 64)).astype(np.float32)
    nan_row = 3 if shape == "wide" else 1
    if case == "special":
        w[nan_row, :] = np.nan
        w[2, 7] = np.inf
        w[T - 1, :] = -0.0
        w[0, :] = -w[0, :]
        w[T - 2, 11] = -np.inf
    dpool = index_pool_to_device(pool, 64, 128)
    drs, drl, dpt = t_dev(np.arange(T, dtype=np.int32)), t_dev(np.array(lens, np.int32)), t_dev(pt)
    qs = t_dev(qsc.astype(np.float32))
    N = max(lens)
    phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(t_dev(qcodes), t_dev(w), drs, drl, N, dpt, dpool, phys, logi,
                        q_fmt=csa.CSA_FP8_E4M3, q_scale=qs)
    logits = torch.full((T, N), float("nan"), device=DEV)
    csa.indexer_score(t_dev(qcodes), t_dev(w), drs, drl, N, dpt, dpool, logits,
                      q_fmt=csa.CSA_FP8_E4M3, q_scale=qs)
    phys2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    logi2 = torch.empty((T, 512), dtype=torch.int32, device=DEV)
    csa.topk512_page_select(logits, drl, drs, dpt, phys2, logi2)
    gl, wl = logi.cpu().numpy(), logi2.cpu().numpy()
    bad = [t for t in range(T) if not np.array_equal(gl[t], wl[t])]
    assert not bad, f"{len(bad)} rows differ from the two calls, first {bad[:5]}"
    assert np.array_equal(phys.cpu().numpy(), phys2.cpu().numpy())
    lg = logits.cpu().numpy()
    if case == "special":
        assert np.isnan(lg[nan_row, :lens[nan_row]]).all()
        assert np.array_equal(gl[nan_row], np.arange(512))  # all NaN: the lowest indices
    else:
        # each row's selection is the top-512 by (logit desc, index asc) of its logits
        for t in (0, 1, T - 1):
            n = lens[t]
            order = np.lexsort((np.arange(n), -lg[t, :n].astype(np.float64)))[:512]
            assert np.array_equal(gl[t], np.sort(order)), f"row {t}"


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


@pytest.mark.parametrize("fmt,with_rope", [("fp8", False), ("mxfp4", False), ("fp8", True),
                                           ("mxfp4", True)])
def test_decode_prep(csa, fmt, with_rope):
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
    table = _rope_table(int(lens.max()), 64) if with_rope else None
    flags = csa.CSA_PREP_HADAMARD | (csa.CSA_PREP_ROPE if with_rope else 0)
    csa.csa_decode_prep(x, t_dev(pos), t_dev(w), t_dev(b), t_dev(pt), c4, t_dev(pt), raw,
                        k_rows=k, q_rows=q, kpool=kpool, q_out=q_out, q_out_scale=q_sc, flags=flags,
                        rope_table=None if table is None else t_dev(table))

    def rope_of(p, n):
        """The oracle's rope argument for n rows at position p (or None)."""
        if table is None:
            return None
        cs = np.repeat(table[p][None].astype(np.float64), n, axis=0)
        return (cs[..., 0], cs[..., 1], 64)
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
        err = Q.compress_error_bound(xh[s], w)
        ok, msg, _ = Q.fp8_rows_match(lat[slot][None], sc[slot:slot + 1], c[:, :512], err[None, :512])
        assert ok, f"sequence {s}: compressed latent: {msg}"
        ok, msg = Q.bf16_match(rope[slot], c[0, 512:], err[512:])
        assert ok, f"sequence {s}: compressed RoPE dims: {msg}"
        ke = Q.exact_rotated(kh[s:s + 1], True, rope=rope_of(int(pos[s]), 1))
        kerr = Q.rotation_error_bound(kh[s:s + 1], 128, rope=with_rope)
        if fmt == "fp8":
            ok, msg, _ = Q.fp8_rows_match(kd[slot][None], ks[slot].view(np.float32), ke, kerr)
        else:
            ok, msg, _ = Q.mxfp4_rows_match(kd[slot][None], ks[slot][None], ke, kerr)
        assert ok, f"sequence {s}: index-K row: {msg}"
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
    qr = qh.reshape(-1, 128)
    match = Q.fp8_rows_match if fmt == "fp8" else Q.mxfp4_rows_match
    qrope = None
    if table is not None:
        cs = table[np.repeat(pos, H_I)].astype(np.float64)
        qrope = (cs[..., 0], cs[..., 1], 64)
    ok, msg, _ = match(q_out.cpu().numpy().reshape(B * H_I, -1), q_sc.cpu().numpy().reshape(B * H_I, -1),
                       Q.exact_rotated(qr, True, rope=qrope), Q.rotation_error_bound(qr, 128, rope=with_rope))
    assert ok, f"query rows: {msg}"


# ------------------------------------------------------------------ generic top-k and DSA mode


@pytest.mark.parametrize("k,lens", [
    (1, [5000, 1, 0, 30000]),
    (100, [99, 100, 101, 16384, 70000]),
    (512, [8192, 200000]),                       # the generic entry at k = 512
    (1000, [999, 5000, 40000, 131072]),
    (2048, [2048, 2049, 16384, 131072]),          # whole rows, chunked rows
    (2048, [500000]),                             # near the longest row k = 2048 takes
])
def test_topk_generic_k_bit_exact(csa, k, lens):
    """topk_page_select for k != 512 (DSA's generic top-k) against the oracle,
    bit for bit: ties (rounded logits), -0 / +0, a NaN, a short row, an empty
    row; slots through a 64-entry page table."""
    g = gen.rng(1400 + k + len(lens))
    R, L = len(lens), max(max(lens), 1)
    pps = (L + 63) // 64
    pt = gen.page_table(g, R, pps, R * pps + 5)
    logits = (np.round(g.standard_normal((R, L)) * 16) / 16).astype(np.float32)
    logits[0, 1:200:3] = -0.0
    logits[-1, 7] = np.nan
    phys = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
    csa.topk_page_select(t_dev(logits), t_dev(np.array(lens, np.int32)), t_dev(np.arange(R, dtype=np.int32)),
                         t_dev(pt), k, phys, logi, page_size=64)
    gp, gl = phys.cpu().numpy(), logi.cpu().numpy()
    for r, n in enumerate(lens):
        wp, wl = O.topk_page_select(logits[r], n, pt[r], 64, k)
        assert np.array_equal(gl[r], wl), f"row {r} (len {n}): logical indices differ"
        assert np.array_equal(gp[r], wp), f"row {r} (len {n}): physical slots differ"


def _kv_pool_chunked(g, n_rows, fmt="fp8", step=1 << 14):
    """An oracle KV pool of n_rows seeded N(0,1) entries, quantised in pieces."""
    parts = [O.quant_kv_entries(gen.normal(g, (min(step, n_rows - r0), 576)), fmt)
             for r0 in range(0, n_rows, step)]
    return O.KVPool(np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]),
                    np.concatenate([p[2] for p in parts]), fmt)


def test_dsa_decode_end_to_end(csa):
    """The DSA (ratio-1) decode step over raw tokens: index-K and KV pools of
    raw tokens in 64-token pages, indexer_score over tokens j <= p,
    topk_page_select with k = 2048, csa_sparse_attn over the selection with no
    window. Logits within 1e-4 of the row max; the selection equal to the
    oracle's top-2048 outside the near-tie band; attention within 2e-2 of the
    oracle's over the GPU's selection."""
    from tests.fullsize import topk_agrees
    g = gen.rng(1500)
    lens = [1500, 20000, 70000]  # raw tokens; the first is shorter than k
    B, k, H = len(lens), 2048, 64
    pps = max((n + 63) // 64 for n in lens)
    P = B * pps + 3
    pt = gen.page_table(g, B, pps, P)
    kdata, ksc = O.index_prep(gen.normal(g, (P * 64, 128)), True, "fp8")
    ipool = O.IndexPool(kdata, ksc, "fp8")
    kv = _kv_pool_chunked(g, P * 64)
    qcodes, qsc = O.index_prep(gen.normal(g, (B, 64, 128)), True, "fp8")
    w = gen.uniform(g, (B, 64))
    q, qh = _bf16(gen.normal(g, (B, H, 576)))
    dpt, rs, rl = t_dev(pt), t_dev(np.arange(B, dtype=np.int32)), t_dev(np.array(lens, np.int32))
    logits = torch.full((B, max(lens)), float("nan"), device=DEV)
    csa.indexer_score(t_dev(qcodes), t_dev(w), rs, rl, max(lens), dpt, index_pool_to_device(ipool, 64, 128),
                      logits, q_fmt=csa.CSA_FP8_E4M3, q_scale=t_dev(qsc.astype(np.float32)))
    phys = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    logi = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    csa.topk_page_select(logits, rl, rs, dpt, k, phys, logi, page_size=64)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    dkv = kv_pool_to_device(kv, 64)
    csa.csa_sparse_attn(q, rs, t_dev(np.array(lens, np.int32) - 1), phys, dkv, dkv, dpt, 0, 576 ** -0.5, out)
    gl_, gp, gq = logits.cpu().numpy(), phys.cpu().numpy(), logi.cpu().numpy()
    go = out.float().cpu().numpy()
    qhat = O.dequant_fp8_rows(qcodes, qsc)
    for b, n in enumerate(lens):
        o_logits, o_sel, _ = O.dsa_query(qhat[b], w[b], ipool, kv, pt[b], n - 1, qh[b], k, 576 ** -0.5)
        tol = 1e-4 * np.abs(o_logits).max()
        assert np.abs(gl_[b, :n] - o_logits).max() <= tol, f"seq {b}: logits"
        ok, _, nband = topk_agrees(o_logits, gq[b], k, tol)
        assert ok, f"seq {b}: top-{k} differs outside the near-tie band ({nband} in band)"
        sel = gq[b][gq[b] >= 0]
        assert np.array_equal(gp[b][:len(sel)], O.page_slot(pt[b], sel, 64))
        want = O.attend(qh[b], kv.rows(O.page_slot(pt[b], sel, 64)), 576 ** -0.5)
        assert np.abs(go[b] - want).max() <= 2e-2, f"seq {b}: attention"


def test_hisparse_swap_in_against_oracle(csa):
    """HiSparse staging over six steps of overlapping selections (three
    sequences, 1024 hot slots, top-512): near-pool slots, the residency maps
    and stamps equal the oracle's exactly; the staged rows equal the far
    pool's bytes; attention over the near pool equals attention over the far
    pool bit for bit."""
    g = gen.rng(1600)
    S, N, hot, k = 3, 20000, 1024, 512
    pps = (N + 63) // 64
    P = S * pps + 2
    pt = gen.page_table(g, S, pps, P)
    far = _kv_pool_chunked(g, P * 64)
    dfar = kv_pool_to_device(far, 64)
    near = csa.alloc_kv_pool(S * hot // 64, 64, csa.CSA_FP8_E4M3)
    slot_of = torch.full((S, N), -1, dtype=torch.int32, device=DEV)
    owner = torch.full((S, hot), -1, dtype=torch.int32, device=DEV)
    last_use = torch.zeros((S, hot), dtype=torch.int32, device=DEV)
    states = [O.HotSet(hot) for _ in range(S)]
    rs = t_dev(np.arange(S, dtype=np.int32))
    dpt = t_dev(pt)
    q, _ = _bf16(gen.normal(g, (S, 64, 576)))
    prev = [np.sort(g.choice(N, size=k, replace=False)) for _ in range(S)]
    for step in range(6):
        sel = np.full((S, k), -1, np.int32)
        for s in range(S):
            keep = prev[s][g.random(len(prev[s])) < 0.7]
            new = g.choice(N, size=k, replace=False)
            cur = np.unique(np.concatenate([keep, new]))[:k]
            if s == 2 and step % 2:
                cur = cur[:300]  # a short selection, -1 padded
            cur = np.sort(cur)
            sel[s, :len(cur)] = cur
            prev[s] = cur
        near_idx = torch.full((S, k), -7, dtype=torch.int32, device=DEV)
        csa.hisparse_swap_in(t_dev(sel), rs, dfar, dpt, near, hot, slot_of, owner, last_use, step, near_idx)
        torch.cuda.synchronize()
        gn = near_idx.cpu().numpy()
        for s in range(S):
            want, _ = O.hisparse_swap_in(states[s], [int(j) for j in sel[s]], step)
            want = np.array([s * hot + h if h >= 0 else -1 for h in want])
            assert np.array_equal(gn[s], want), f"step {step} seq {s}: near slots differ"
            own = owner[s].cpu().numpy()
            assert np.array_equal(own, np.array(states[s].owner)), f"step {step} seq {s}: owners"
            assert np.array_equal(last_use[s].cpu().numpy(), np.array(states[s].last_use))
            so = slot_of[s].cpu().numpy()
            res = np.flatnonzero(so >= 0)
            assert sorted(res.tolist()) == sorted(states[s].slot_of.keys())
            assert all(so[j] == states[s].slot_of[j] for j in res)
        # the staged rows are the far rows of the selected entries
        ok = sel >= 0
        fslots = np.where(ok, np.stack([O.page_slot(pt[s], np.maximum(sel[s], 0), 64) for s in range(S)]), 0)
        nl = near.latent.view(-1, 512).cpu().numpy()
        ns = near.scale.view(-1).cpu().numpy()
        nr = near.rope.view(-1, 64).cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(nl[gn[ok]], far.latent[fslots[ok]])
        assert np.array_equal(ns[gn[ok]], far.scale[fslots[ok]])
        assert np.array_equal(nr[gn[ok]], far.rope[fslots[ok]])
        # attention over the near pool == over the far pool (same rows, same order)
        pos = t_dev(np.full(S, 4 * N, np.int32))
        o_near = torch.empty((S, 64, 512), dtype=torch.bfloat16, device=DEV)
        o_far = torch.empty((S, 64, 512), dtype=torch.bfloat16, device=DEV)
        csa.csa_sparse_attn(q, rs, pos, near_idx, near, near, dpt, 0, 576 ** -0.5, o_near)
        csa.csa_sparse_attn(q, rs, pos, t_dev(np.where(ok, fslots, -1).astype(np.int32)), dfar, dfar, dpt,
                            0, 576 ** -0.5, o_far)
        assert torch.equal(o_near.view(torch.int16), o_far.view(torch.int16)), f"step {step}: attention"
