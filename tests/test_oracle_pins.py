"""Pins of the CPU oracle against facts fixed by the pages, by published format
specifications and by mathematics -- never against the oracle itself.

Each test names what it pins. Sources: [P1] "Token 的一生：DSV4 架构与 DSpark";
[P2] "DeepSeek-V4 的交錯壓縮注意力（CSA/HCA）：將百萬標記長上下文變為可用資源".
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

from oracle import csa_oracle as O
from tests.conftest import read_golden

# ---------------------------------------------------------------- constants


def test_constants_match_pages():
    consts = {ln.split()[0]: int(ln.split()[1]) for ln in read_golden("constants.txt")}
    assert consts["c4_ratio"] == 4
    assert consts["raw_page_size"] == O.RAW_PAGE
    assert consts["c4_page_size"] == O.C4_PAGE == consts["raw_page_size"] // consts["c4_ratio"]
    assert consts["topk"] == O.TOPK
    assert consts["kv_rope_dims"] == O.ROPE_DIM and O.LATENT_DIM + O.ROPE_DIM == O.KV_DIM


# ---------------------------------------------------------------- FP8 e4m3fn


def test_e4m3_table_matches_torch_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.E4M3_VALUES
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(ours[finite], ref[finite])
    assert O.E4M3_VALUES[0x7E] == 448.0 and O.E4M3_VALUES[1] == 2.0 ** -9


def test_e4m3_encode_matches_torch_cast():
    """torch's CPU cast is round-to-nearest-even but does not saturate, so the
    input is clamped to +-448 first (the saturation the reading adopts)."""
    g = np.random.default_rng(7)
    v = np.concatenate([
        g.standard_normal(200000) * 100,
        g.standard_normal(50000) * 1e-3,            # subnormal range
        O.E4M3_VALUES[np.isfinite(O.E4M3_VALUES)],  # exact codes
        (O.E4M3_VALUES[1:126] + O.E4M3_VALUES[2:127]) / 2,  # exact midpoints (ties)
        [0.0, -0.0, 447.9, 448.0, 449.0, -1e9, 1e9],
    ]).astype(np.float32)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), ref)


def test_e4m3_roundtrip_all_codes():
    vals = O.E4M3_VALUES
    codes = np.arange(256, dtype=np.uint8)
    finite = np.isfinite(vals)
    assert np.array_equal(O.e4m3_encode(vals[finite]), codes[finite])


def test_quant_fp8_rows_scale_and_error_bound():
    g = np.random.default_rng(3)
    v = g.standard_normal((64, 128)).astype(np.float32)
    codes, scale = O.quant_fp8_rows(v)
    amax = np.abs(v).max(axis=1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    # the largest element maps to (about) 448; relative error of e4m3 RNE <= 2^-4
    deq = O.dequant_fp8_rows(codes, scale)
    big = np.abs(v) >= scale[:, None] * 2 ** -6  # normal range of e4m3
    assert np.all(np.abs(deq - v)[big] <= np.abs(v)[big] * 2 ** -4 * (1 + 1e-6))
    assert np.all(np.abs(deq - v)[~big] <= (scale[:, None] * 2 ** -10 * (1 + 1e-6)).repeat(128, 1)[~big])


def test_bf16_matches_torch_cast():
    g = np.random.default_rng(5)
    v = np.concatenate([g.standard_normal(100000), g.standard_normal(1000) * 1e-30,
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_bits(v), ref)
    assert np.array_equal(O.bf16_decode(ref), torch.from_numpy(v).to(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- MXFP4


def test_e2m1_table_matches_ocp_spec():
    rows = [ln.split() for ln in read_golden("e2m1_codes.txt")]
    table = {int(c): float(v) for c, v in rows}
    for code in range(8):
        assert O.E2M1_VALUES[code] == table[code]
        assert -O.E2M1_VALUES[code] == table[code + 8]


def test_mxfp4_hand_worked_blocks():
    for ln in read_golden("mxfp4_blocks.txt"):
        vals, sbyte, codes, decoded = [p.split() for p in ln.split("|")]
        v = np.zeros(32, dtype=np.float32)
        v[:4] = [float(x) for x in vals]
        packed, sc = O.quant_mxfp4_rows(v[None])
        unpacked = np.empty(32, dtype=np.uint8)
        unpacked[0::2] = packed[0] & 0xF
        unpacked[1::2] = packed[0] >> 4
        assert int(sc[0, 0]) == int(sbyte[0])
        assert [int(c) for c in unpacked[:4]] == [int(c) for c in codes]
        # and back: the stored bytes decode to the hand-worked values, sign of zero included
        deq = O.dequant_mxfp4_rows(packed, sc)[0]
        want = np.array([float(x) for x in decoded])
        assert np.array_equal(deq[:4], want) and np.array_equal(np.signbit(deq[:4]), np.signbit(want))
        assert np.all(deq[4:] == 0.0)


def test_mxfp4_decode_hand_decoded_bytes():
    """Bytes decoded by hand from the OCP MX v1.0 definitions (fixture): fixes
    the nibble order, the sign bit and the e8m0 bias, extremes included."""
    for ln in read_golden("mxfp4_decode.txt"):
        hexes, sbyte, vals = [p.split() for p in ln.split("|")]
        n = len(hexes)
        packed = np.zeros(16, dtype=np.uint8)
        packed[:n] = [int(h, 16) for h in hexes]
        deq = O.dequant_mxfp4_rows(packed[None], np.array([[int(sbyte[0])]], dtype=np.uint8))[0]
        want = np.array([float(x) for x in vals])
        assert np.array_equal(deq[:2 * n], want), (ln, deq[:2 * n])
        assert np.array_equal(np.signbit(deq[:2 * n]), np.signbit(want))


def test_mxfp4_decode_every_code_and_scale():
    """All 16 e2m1 codes in both nibble positions, times 2^(byte - 127) for
    e8m0 bytes across the range, against the OCP table of the fixture."""
    table = {int(c): float(v) for c, v in (ln.split() for ln in read_golden("e2m1_codes.txt"))}
    for byte in (0, 1, 100, 126, 127, 128, 131, 200, 253, 254):
        for c in range(16):
            packed = np.zeros((1, 16), dtype=np.uint8)
            packed[0, 0] = c | ((15 - c) << 4)   # element 0 = c, element 1 = 15 - c
            packed[0, 5] = (c << 4) | 0x1        # element 10 = 0.5, element 11 = c
            deq = O.dequant_mxfp4_rows(packed, np.array([[byte]], dtype=np.uint8))[0]
            sc = math.ldexp(1.0, byte - 127)
            assert deq[0] == table[c] * sc and deq[1] == table[15 - c] * sc
            assert deq[10] == 0.5 * sc and deq[11] == table[c] * sc
            assert np.signbit(deq[0]) == (c >= 8)


def test_mxfp4_roundtrip_error_bound():
    """quant then dequant: within half a grid step of the value (the e2m1 grid
    at scale 2^X has steps 0.5, 1, 2 below 2, 4, 6), except values beyond
    6 * 2^X, which saturate to +-6 * 2^X."""
    g = np.random.default_rng(31)
    v = (g.standard_normal((400, 128)) * np.exp(g.uniform(-6, 6, (400, 1)))).astype(np.float32)
    packed, sc = O.quant_mxfp4_rows(v)
    deq = O.dequant_mxfp4_rows(packed, sc)
    X = np.repeat(sc.astype(np.float64) - 127, 32, axis=1)
    a = np.abs(v.astype(np.float64)) / np.exp2(X)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * np.exp2(X)
    sat = a > 6
    err = np.abs(deq - v)
    assert np.all(err[~sat] <= half[~sat])
    assert np.array_equal(np.abs(deq[sat]), 6 * np.exp2(X[sat]))
    assert np.all(np.sign(deq[deq != 0]) == np.sign(v[deq != 0]))


def test_mxfp4_brute_force_nearest_even():
    """Every element code is the nearest e2m1 value to v / 2^X (ties to the even
    code), checked by exhaustive search over the 8 magnitudes."""
    g = np.random.default_rng(11)
    v = (g.standard_normal((300, 128)) * np.exp(g.uniform(-8, 8, (300, 1)))).astype(np.float32)
    v[0, :32] = 0.0  # all-zero block
    packed, sc = O.quant_mxfp4_rows(v)
    X = sc.astype(np.int64) - 127
    code = np.empty(v.shape, dtype=np.uint8)
    code[:, 0::2] = packed & 0xF
    code[:, 1::2] = packed >> 4
    for r in range(0, 300, 7):
        for blk in range(4):
            x = X[r, blk]
            seg = v[r, blk * 32:(blk + 1) * 32].astype(np.float64)
            amax = np.abs(seg).max()
            if amax == 0:
                assert x == -127
            else:
                assert 2.0 ** (x + 2) <= amax < 2.0 ** (x + 3)  # top binade of e2m1 (4 <= amax/2^X < 8)
            for i, val in enumerate(seg):
                target = min(abs(val) / 2.0 ** x, 6.0)
                d = np.abs(O.E2M1_VALUES - target)
                best = np.flatnonzero(d == d.min())
                best = best[best % 2 == 0][0] if len(best) > 1 else best[0]
                c = code[r, blk * 32 + i]
                assert (c & 7) == best
                assert bool(c & 8) == bool(np.signbit(val))
    deq = O.dequant_mxfp4_rows(packed, sc)
    assert np.all(np.abs(deq) <= 6.0 * np.exp2(X).repeat(32, axis=1))


# ---------------------------------------------------------------- Hadamard ([P1] §4)


@pytest.mark.parametrize("D", [2, 8, 64, 128])
def test_hadamard_equals_sylvester_matrix(D):
    g = np.random.default_rng(D)
    v = g.standard_normal((5, D))
    H = scipy.linalg.hadamard(D).astype(np.float64)  # Sylvester construction
    np.testing.assert_allclose(O.hadamard_rotate(v), v @ H.T / math.sqrt(D), rtol=0, atol=1e-12)
    assert np.array_equal(H @ H.T, D * np.eye(D))


def test_hadamard_preserves_scores():
    """Rotating both q and k leaves unquantised indexer logits unchanged."""
    g = np.random.default_rng(1)
    q = g.standard_normal((64, 128))
    k = g.standard_normal((300, 128))
    w = g.uniform(0, 1, 64)
    a = O.indexer_logits(q, w, k)
    b = O.indexer_logits(O.hadamard_rotate(q), w, O.hadamard_rotate(k))
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-9)


def test_index_prep_rotates_exactly_then_rounds_once():
    """index_prep with the Hadamard flag and 'f32' output is the float32
    rounding of the exact product with scipy's Sylvester matrix (library
    routine), and the quantised formats quantise that float32 value."""
    g = np.random.default_rng(44)
    v = g.standard_normal((300, 128)).astype(np.float32)
    exact = v.astype(np.float64) @ scipy.linalg.hadamard(128).T / math.sqrt(128)
    got, _ = O.index_prep(v, True, "f32")
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got, exact.astype(np.float32))
    c, s = O.index_prep(v, True, "fp8")
    c2, s2 = O.quant_fp8_rows(exact.astype(np.float32))
    assert np.array_equal(c, c2) and np.array_equal(s, s2)


# ---------------------------------------------------------------- RoPE ([P1] §3.1, §4)


def _rot2(angle):
    return np.array([[math.cos(angle), -math.sin(angle)], [math.sin(angle), math.cos(angle)]])


def test_rope_worked_example_and_layout():
    """One pair rotated by a quarter turn: (1, 0) -> (0, 1), (0, 1) -> (-1, 0)
    (counter-clockwise, x' = x cos - y sin); only the last rope_dim dims move."""
    v = np.array([[5.0, 7.0, 1.0, 0.0], [5.0, 7.0, 0.0, 1.0]])
    out = O.rope_rotate(v, np.array([[0.0], [0.0]]), np.array([[1.0], [1.0]]), 2)
    np.testing.assert_array_equal(out, [[5.0, 7.0, 0.0, 1.0], [5.0, 7.0, -1.0, 0.0]])


def test_rope_frequencies_closed_form():
    """Angle of pair i at position p is p * theta^(-2i/d): pair 0 turns by p
    radians, the angles form a geometric sequence of ratio theta^(-2/d)."""
    cos, sin = O.rope_cos_sin([0, 1, 3, 1000], 64, 10000.0)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)  # position 0: identity
    ang = np.arctan2(sin[1], cos[1])
    np.testing.assert_allclose(ang, 10000.0 ** (-np.arange(32) / 32), rtol=1e-13)
    assert sin[2, 0] == math.sin(3.0) and cos[2, 0] == math.cos(3.0)


def test_rope_matches_explicit_block_rotation_matrix():
    """rope_rotate equals the block-diagonal matrix of 2 x 2 rotations acting
    on the last rope_dim dims (pairs of adjacent dims)."""
    g = np.random.default_rng(45)
    D, rd = 128, 64
    v = g.standard_normal((6, D))
    pos = np.array([0, 1, 5, 4095, 131071, 1048575])
    cos, sin = O.rope_cos_sin(pos, rd)
    got = O.rope_rotate(v, cos, sin, rd)
    for r, p in enumerate(pos):
        M = np.eye(D)
        for i in range(rd // 2):
            a = p * 10000.0 ** (-2 * i / rd)
            M[D - rd + 2 * i:D - rd + 2 * i + 2, D - rd + 2 * i:D - rd + 2 * i + 2] = _rot2(a)
        np.testing.assert_allclose(got[r], M @ v[r], rtol=1e-9, atol=1e-9)


def test_rope_norm_and_relative_position():
    """Rotations preserve the norm, and a rotated query and key interact only
    through their position difference: (R_m q) . (R_n k) = (R_{m-n} q) . k."""
    g = np.random.default_rng(46)
    q = g.standard_normal((50, 128))
    k = g.standard_normal((50, 128))
    m = g.integers(0, 1 << 20, 50)
    n = g.integers(0, 1 << 20, 50)
    cm, sm = O.rope_cos_sin(m, 64)
    cn, sn = O.rope_cos_sin(n, 64)
    cd, sd = O.rope_cos_sin(m - n, 64)
    qm = O.rope_rotate(q, cm, sm, 64)
    np.testing.assert_allclose(np.linalg.norm(qm, axis=1), np.linalg.norm(q, axis=1), rtol=1e-12)
    lhs = (qm * O.rope_rotate(k, cn, sn, 64)).sum(1)
    rhs = (O.rope_rotate(q, cd, sd, 64) * k).sum(1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-7, atol=1e-7)


def test_index_prep_order_rope_then_hadamard():
    """[P1] §4 fixes the order rope -> hadamard -> quant: index_prep with both
    equals H (R v) / sqrt(D), which differs from R (H v) / sqrt(D)."""
    g = np.random.default_rng(47)
    v = g.standard_normal((20, 128))
    pos = g.integers(1, 5000, 20)
    cos, sin = O.rope_cos_sin(pos, 64)
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    Rv = np.stack([np.concatenate([v[r, :64]] + [
        _rot2(p * 10000.0 ** (-2 * i / 64)) @ v[r, 64 + 2 * i:66 + 2 * i] for i in range(32)])
        for r, p in enumerate(pos)])
    got, _ = O.index_prep(v, True, "f32", rope=(cos, sin, 64))
    np.testing.assert_array_equal(got, (Rv @ H.T).astype(np.float32))
    other = O.rope_rotate(v @ H.T, cos, sin, 64).astype(np.float32)
    assert not np.allclose(got, other, atol=1e-3)


# ---------------------------------------------------------------- compressor ([P1] §2.1, [P2])


def test_compress_uniform_gate_is_block_mean():
    g = np.random.default_rng(2)
    x = g.standard_normal((64, 576))
    out = O.compress_blocks(x, 0, 4, np.zeros(576), np.full(4, 0.37))
    np.testing.assert_allclose(out, x.reshape(16, 4, 576).mean(axis=1), rtol=0, atol=1e-14)


def test_compress_closed_form_bias_weights():
    g = np.random.default_rng(4)
    for ln in read_golden("compress_closed_form.txt"):
        r, ms = ln.split("|")
        ratio = int(r)
        m = np.array([float(t) for t in ms.split()])
        x = g.standard_normal((3 * ratio, 576))
        out = O.compress_blocks(x, 8, ratio, np.zeros(576), np.log(m))
        want = (m[None, :, None] * x.reshape(3, ratio, 576)).sum(axis=1) / m.sum()
        np.testing.assert_allclose(out, want, rtol=0, atol=1e-13)


def test_compress_one_hot_limit_and_bias_position():
    """A bias of +60 on position i of the block selects row i (to e^-60)."""
    g = np.random.default_rng(6)
    x = g.standard_normal((40, 576))
    for i in range(4):
        b = np.zeros(4)
        b[i] = 60.0
        out = O.compress_blocks(x, 0, 4, np.zeros(576), b)
        np.testing.assert_allclose(out, x[i::4], rtol=0, atol=1e-20 + 1e-24 + 1e-12)


def test_compress_data_term_and_shift_invariance():
    g = np.random.default_rng(8)
    x = g.standard_normal((16, 576))
    w = g.standard_normal(576) / 24
    b = g.standard_normal(4) * 0.3
    a = O.compress_blocks(x, 4, 4, w, b)
    np.testing.assert_allclose(a, O.compress_blocks(x, 4, 4, w, b + 5.0), rtol=1e-12, atol=1e-14)
    # the data term: doubling w on rows whose gates differ changes the result
    assert not np.allclose(a, O.compress_blocks(x, 4, 4, 2 * w, b))
    # explicit two-row check of the gate: softmax of w.x_i + b_i
    g0 = x[4:8] @ w + b
    p = np.exp(g0 - g0.max())
    p /= p.sum()
    np.testing.assert_allclose(a[1], p @ x[4:8], rtol=1e-12)
    # partial tail block is not compressed
    assert O.compress_blocks(x[:7], 0, 4, w, b).shape == (1, 576)


def test_compress_ratio_one_is_identity():
    g = np.random.default_rng(9)
    x = g.standard_normal((10, 576))
    np.testing.assert_array_equal(O.compress_blocks(x, 3, 1, g.standard_normal(576), [0.5]), x)


def test_hca_ratio_128_mean():
    g = np.random.default_rng(10)
    x = g.standard_normal((300, 576))
    out = O.compress_blocks(x, 0, 128, np.zeros(576), np.zeros(128))
    assert out.shape == (2, 576)
    np.testing.assert_allclose(out, x[:256].reshape(2, 128, 576).mean(axis=1), atol=1e-13)


def test_kv_entry_storage():
    g = np.random.default_rng(12)
    c = g.standard_normal((20, 576))
    lat, sc, rp = O.quant_kv_entries(c, "fp8")
    assert lat.shape == (20, 512) and sc.shape == (20,) and rp.shape == (20, 64)
    deq = O.dequant_kv_entries(lat, sc, rp, "fp8")
    np.testing.assert_allclose(deq[:, 512:], c[:, 512:], rtol=2 ** -8)
    assert np.all(np.abs(deq[:, :512] - c[:, :512]) <= np.maximum(np.abs(c[:, :512]) * 2 ** -4, sc[:, None] * 2 ** -9) * 1.0001)


# ---------------------------------------------------------------- indexer ([P1] §3, [P2])


def test_indexer_single_head_is_relu_dot():
    g = np.random.default_rng(13)
    q = g.standard_normal((1, 64))
    k = g.standard_normal((50, 64))
    np.testing.assert_allclose(O.indexer_logits(q, [1.0], k), np.maximum(k @ q[0], 0), rtol=1e-13)


def test_indexer_relu_per_head_before_weighting():
    """Two heads with q.k = 2 and -3, weights 1 and 1: the score is 2
    (ReLU per head, then the weighted sum), not -1 and not 5."""
    k = np.array([[1.0, 0.0]])
    q = np.array([[2.0, 0.0], [-3.0, 0.0]])
    assert O.indexer_logits(q, [1.0, 1.0], k)[0] == 2.0
    assert O.indexer_logits(q, [0.5, 7.0], k)[0] == 1.0


def test_indexer_scale_factoring():
    """ReLU(a x) = a ReLU(x) for a > 0: folding a positive q scale into w."""
    g = np.random.default_rng(14)
    q = g.standard_normal((8, 64))
    k = g.standard_normal((30, 64))
    w = g.uniform(0, 1, 8)
    a = g.uniform(0.1, 3, 8)
    np.testing.assert_allclose(O.indexer_logits(q * a[:, None], w, k), O.indexer_logits(q, w * a, k), rtol=1e-12)


# ---------------------------------------------------------------- top-512 ([P1] §3.2)


def test_topk_short_row_selects_everything():
    g = np.random.default_rng(15)
    for n in (0, 1, 100, 512):
        logits = g.standard_normal(n)
        assert np.array_equal(O.topk_logical(logits, n), np.arange(n))
        phys, logical = O.topk_page_select(logits, n, np.arange(16))
        assert np.array_equal(logical[:n], np.arange(n)) and np.all(logical[n:] == -1)
        assert np.array_equal(phys, logical)  # identity page table


def test_topk_all_equal_takes_lowest_indices():
    assert np.array_equal(O.topk_logical(np.full(2000, 3.5), 2000), np.arange(512))


def test_topk_equals_stable_argsort():
    g = np.random.default_rng(16)
    for n in (513, 1000, 4096, 33000):
        logits = np.round(g.standard_normal(n) * 8) / 8  # many ties
        ref = np.sort(np.argsort(-logits, kind="stable")[:512])
        assert np.array_equal(O.topk_logical(logits, n), ref)


def test_topk_signed_zero_nan_and_inf():
    v = np.zeros(1000)
    v[::2] = -0.0
    assert np.array_equal(O.topk_logical(v, 1000), np.arange(512))  # -0 == +0
    v = np.full(600, -np.inf)
    v[:90] = 1.0
    v[100] = np.nan
    sel = O.topk_logical(v, 600)
    assert 100 not in sel and len(sel) == 512 and set(range(90)) <= set(sel)
    assert np.array_equal(sel[90:], np.array([j for j in range(90, 600) if j != 100][:422]))


@pytest.mark.parametrize("k", [1, 100, 2048])
def test_topk_generic_k_equals_stable_argsort(k):
    """The generic top-k (DSA's selection) is the first k of a stable argsort
    by descending logit; k = 1 is the first index of the maximum."""
    g = np.random.default_rng(160 + k)
    for n in (k, k + 1, 3 * k + 5, 40000):
        logits = np.round(g.standard_normal(n) * 6) / 6
        ref = np.sort(np.argsort(-logits, kind="stable")[:k])
        assert np.array_equal(O.topk_logical(logits, n, k), ref)
    v = np.array([1.0, 3.0, -2.0, 3.0])
    assert np.array_equal(O.topk_logical(v, 4, 1), [1])


def test_topk_respects_row_len():
    v = np.arange(3000, dtype=np.float64)
    assert np.array_equal(O.topk_logical(v, 1000), np.arange(488, 1000))


def test_page_table_identity_and_permutation_covariance():
    g = np.random.default_rng(17)
    n = 64 * 20
    logits = g.standard_normal(n)
    phys, logical = O.topk_page_select(logits, n, np.arange(20))
    assert np.array_equal(phys, logical)
    perm = g.permutation(40)[:20]
    phys2, logical2 = O.topk_page_select(logits, n, perm)
    assert np.array_equal(logical2, logical)
    assert np.array_equal(phys2, perm[logical // 64] * 64 + logical % 64)


# ---------------------------------------------------------------- attention ([P1] §1, [P2])


def _sdpa(q, kv, scale):
    """Library reference: torch's CPU scaled_dot_product_attention in float64."""
    qt = torch.from_numpy(q)[None]
    kt = torch.from_numpy(kv)[None]
    vt = torch.from_numpy(np.ascontiguousarray(kv[:, :512]))[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0].numpy()


def test_attention_matches_sdpa():
    g = np.random.default_rng(18)
    q = g.standard_normal((16, 576))
    kv = g.standard_normal((300, 576))
    s = 576 ** -0.5
    np.testing.assert_allclose(O.attend(q, kv, s), _sdpa(q, kv, s), rtol=1e-10, atol=1e-12)


def test_attention_single_entry_and_convex_hull():
    g = np.random.default_rng(19)
    q = g.standard_normal((4, 576))
    kv = g.standard_normal((1, 576))
    np.testing.assert_allclose(O.attend(q, kv, 0.04), np.repeat(kv[:, :512], 4, 0), atol=1e-15)
    kv = g.standard_normal((50, 576))
    o = O.attend(q, kv, 0.5)
    assert np.all(o <= kv[:, :512].max(0) + 1e-12) and np.all(o >= kv[:, :512].min(0) - 1e-12)


def _mk_pools(g, n_c4, n_raw, fmt="f32", idx_fmt="f32", D=64):
    c = g.standard_normal((n_c4, 576))
    r = g.standard_normal((n_raw, 576))
    c4 = O.KVPool(*O.quant_kv_entries(c, fmt), fmt)
    raw = O.KVPool(*O.quant_kv_entries(r, fmt), fmt)
    k = g.standard_normal((n_c4, D))
    data, sc = O.index_prep(k, idx_fmt != "f32", idx_fmt)
    return c4, raw, O.IndexPool(data, sc, idx_fmt)


def test_csa_short_context_equals_dense_attention():
    """c4 length <= 512: top-512 keeps everything, so CSA is dense attention
    over all compressed entries plus the window (the method's special case)."""
    g = np.random.default_rng(20)
    L = 1800
    n = L // 4
    c4, raw, ip = _mk_pools(g, 64 * 8, 256 * 8)
    pt = np.arange(8)
    q_idx = g.standard_normal((8, 64))
    w = g.uniform(0, 1, 8)
    q = g.standard_normal((16, 576))
    s = 576 ** -0.5
    _, sel, out = O.csa_query(q_idx, w, ip, c4, raw, pt, pt, n, L - 1, q, 128, s)
    assert np.array_equal(sel, np.arange(n))
    kv = np.concatenate([c4.rows(np.arange(n)), raw.rows(np.arange(L - 128, L))])
    np.testing.assert_allclose(out, _sdpa(q, kv, s), rtol=1e-10, atol=1e-12)


def test_csa_brute_force_masked_attention():
    """Brute force: score every compressed entry, mask the unselected ones to
    -inf, softmax with the window, compare. Uses a random page table."""
    g = np.random.default_rng(21)
    L = 4096 + 4 * 37 + 2  # ragged tail
    n = L // 4
    pages = (L + 255) // 256
    c4, raw, ip = _mk_pools(g, 64 * 40, 256 * 40, fmt="fp8", idx_fmt="fp8", D=128)
    pt = g.permutation(40)[:pages]
    q_idx_codes, q_sc = O.index_prep(g.standard_normal((64, 128)), True, "fp8")
    q_hat = O.dequant_fp8_rows(q_idx_codes, q_sc)
    w = g.uniform(0, 1, 64)
    q = g.standard_normal((8, 576))
    s = 576 ** -0.5
    logits, sel, out = O.csa_query(q_hat, w, ip, c4, raw, pt, pt, n, L - 1, q, 128, s)
    allk = c4.rows(O.page_slot(pt, np.arange(n), 64))
    scores = s * q @ allk.T
    mask = np.full(n, -np.inf)
    order = sorted(range(n), key=lambda j: (-logits[j], j))[:512]
    mask[order] = 0.0
    win = raw.rows(O.page_slot(pt, np.arange(L - 128, L), 256))
    full = np.concatenate([scores + mask, s * q @ win.T], axis=1)
    p = np.exp(full - full.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    want = p @ np.concatenate([allk, win])[:, :512]
    np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-12)


def test_hca_short_context_is_window_only():
    g = np.random.default_rng(22)
    c4, raw, _ = _mk_pools(g, 64, 256)
    q = g.standard_normal((4, 576))
    pt = np.array([0])
    out = O.hca_query(c4, raw, pt, pt, 100, 128, q, 128, 0.05)
    np.testing.assert_allclose(out, _sdpa(q, raw.rows(np.arange(101)), 0.05), rtol=1e-10, atol=1e-12)


def test_hca_at_ratio_4_equals_csa_when_short():
    """Cross-mode: dense attention over all ratio-4 entries equals CSA when the
    c4 length is <= 512 (everything selected)."""
    g = np.random.default_rng(23)
    c4, raw, ip = _mk_pools(g, 64 * 8, 256 * 8)
    pt = np.arange(8)
    L = 2000
    q = g.standard_normal((8, 576))
    _, _, a = O.csa_query(g.standard_normal((8, 64)), g.uniform(0, 1, 8), ip, c4, raw, pt, pt,
                          L // 4, L - 1, q, 128, 0.04)
    b = O.hca_query(c4, raw, pt, pt, L - 1, 4, q, 128, 0.04)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_prefill_query_equals_decode_at_that_length():
    """Causal visibility 4j+3 <= p: a prefill query at p sees exactly the
    entries a decode step with L = p+1 sees."""
    for p in (0, 2, 3, 4, 7, 130, 131075):
        n_vis = O.causal_row_len(p, 10 ** 9)
        assert all(4 * j + 3 <= p for j in range(max(0, n_vis - 3), n_vis))
        assert 4 * n_vis + 3 > p
        assert n_vis == (p + 1) // 4
    assert O.causal_row_len(131075, 33792) == 32769
    assert O.hca_visible(127, 128) == 1 and O.hca_visible(126, 128) == 0


# ---------------------------------------------------------------- DSA mode ([P1] §1, §2.2)


def test_dsa_short_context_is_dense_causal_attention():
    """k >= p + 1: every visible raw token is selected, so the DSA query is
    dense attention over tokens 0..p (torch SDPA in float64)."""
    g = np.random.default_rng(50)
    n_tok = 64 * 6
    kv, _, ip = _mk_pools(g, n_tok, 64, fmt="fp8", idx_fmt="fp8", D=128)
    pt = g.permutation(6)
    p = 300
    qc, qs = O.index_prep(g.standard_normal((64, 128)), True, "fp8")
    q = g.standard_normal((16, 576))
    logits, sel, out = O.dsa_query(O.dequant_fp8_rows(qc, qs), g.uniform(0, 1, 64), ip, kv, pt, p, q,
                                   2048, 0.05)
    assert len(logits) == p + 1 and np.array_equal(sel, np.arange(p + 1))
    rows = kv.rows(O.page_slot(pt, np.arange(p + 1), 64))
    np.testing.assert_allclose(out, _sdpa(q, rows, 0.05), rtol=1e-10, atol=1e-12)


def test_dsa_brute_force_masked_attention():
    """Brute force: score every visible token, keep the k best by (logit
    descending, index ascending) through an explicit sort, mask the rest to
    -inf, softmax, compare (random 64-token page table, k = 100)."""
    g = np.random.default_rng(51)
    kv, _, ip = _mk_pools(g, 64 * 10, 64, fmt="fp8", idx_fmt="fp8", D=128)
    pt = g.permutation(10)
    p, k = 575, 100
    qc, qs = O.index_prep(g.standard_normal((64, 128)), True, "fp8")
    qhat = O.dequant_fp8_rows(qc, qs)
    w = g.uniform(0, 1, 64)
    q = g.standard_normal((8, 576))
    logits, sel, out = O.dsa_query(qhat, w, ip, kv, pt, p, q, k, 0.04)
    allrows = kv.rows(O.page_slot(pt, np.arange(p + 1), 64))
    order = sorted(range(p + 1), key=lambda j: (-logits[j], j))[:k]
    mask = np.full(p + 1, -np.inf)
    mask[order] = 0.0
    sc = 0.04 * q @ allrows.T + mask
    pr = np.exp(sc - sc.max(1, keepdims=True))
    pr /= pr.sum(1, keepdims=True)
    np.testing.assert_allclose(out, pr @ allrows[:, :512], rtol=1e-10, atol=1e-12)
    assert np.array_equal(sel, np.sort(order))


# ---------------------------------------------------------------- HiSparse ([P1] §5)


def test_hisparse_hand_worked_steps():
    st = O.HotSet(4)
    for ln in read_golden("hisparse_lru.txt"):
        step, sel, near, copies = [p.split() for p in ln.split("|")]
        got_near, got_copies = O.hisparse_swap_in(st, [int(x) for x in sel], int(step[0]))
        assert got_near == [int(x) for x in near], ln
        assert got_copies == [tuple(int(v) for v in c.split(":")) for c in copies], ln


def test_hisparse_invariants_over_many_steps():
    """Maps stay inverse, every selected entry is resident after its step, hits
    copy nothing, nothing selected this step is evicted, and a slot is evicted
    only if no older-stamped free slot was left."""
    g = np.random.default_rng(70)
    hot, k = 64, 24
    st = O.HotSet(hot)
    prev = []
    for step in range(40):
        keep = [j for j in prev if g.random() < 0.6]
        new = list(g.choice(400, size=k, replace=False))
        sel = sorted(set(keep + new))[:k]
        sel += [-1] * (k - len(sel))
        before = dict(st.slot_of)
        stamps = list(st.last_use)
        owners = list(st.owner)
        near, copies = O.hisparse_swap_in(st, sel, step)
        assert all(st.owner[h] == j for j, h in st.slot_of.items())
        assert all(j == -1 or st.slot_of[j] == h for j, h in zip(sel, near))
        assert {j for j, _ in copies} == {j for j in sel if j >= 0 and j not in before}
        used = {h for h in near if h >= 0}
        victims = {h for _, h in copies}
        for h in victims:  # an evicted slot is at least as old as every free slot kept
            kept = [x for x in range(hot) if x not in used and x not in victims]
            if owners[h] >= 0:
                assert all(owners[x] >= 0 and stamps[x] >= stamps[h] for x in kept)
        prev = [j for j in sel if j >= 0]


def test_hisparse_attention_over_near_tier_equals_far():
    """Attention over the staged near-tier rows equals attention over the far
    pool's rows of the same selection (the staging only moves entries)."""
    g = np.random.default_rng(71)
    far_c4, raw, _ = _mk_pools(g, 64 * 20, 256 * 2, fmt="fp8")
    pt = g.permutation(20)
    hot = 600
    st = O.HotSet(hot)
    near_lat = np.zeros((hot, 512), np.uint8)
    near_sc = np.zeros(hot, np.float32)
    near_rope = np.zeros((hot, 64), np.uint16)
    q = g.standard_normal((8, 576))
    for step in range(3):
        sel = np.sort(g.choice(64 * 20, size=512, replace=False))
        near, copies = O.hisparse_swap_in(st, list(sel), step)
        for j, h in copies:
            f = O.page_slot(pt, j, 64)
            near_lat[h], near_sc[h], near_rope[h] = far_c4.latent[f], far_c4.scale[f], far_c4.rope[f]
        near_pool = O.KVPool(near_lat, near_sc, near_rope, "fp8")
        a = O.attend(q, near_pool.rows(near), 0.04)
        b = O.attend(q, far_c4.rows(O.page_slot(pt, sel, 64)), 0.04)
        np.testing.assert_array_equal(a, b)
