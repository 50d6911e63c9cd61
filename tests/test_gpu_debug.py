"""Debug mode (csa_set_debug): the checked calls verify on the device the page
ids, lengths, positions and slots they are about to follow and, on a
violation, return CSA_ERR_BOUNDS without launching their kernels.

Every planted violation stays inside the memory the test allocated: the pools
are views of tensors with two spare pages after the declared ones, and the
bad page ids and slots point into those spare pages; a bad length stays inside the
logits tensor's extra rows. So even a call that launched would read and write
only the test's own buffers; what is checked is that it reports and launches
nothing (outputs keep their fill)."""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_helpers import DEV, index_pool_to_device, kv_pool_to_device, t_dev
from tests.test_gpu_parity import _attn_case, _bf16, _index_case
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture()
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_c4_amd as m
    m.csa_set_debug(True)
    yield m
    m.csa_set_debug(False)


def _spare(t):
    """t with two more pages (copies of its first two) after its own, seen
    as a view of its own size."""
    if t is None:
        return None
    return torch.cat([t, t[:2]]).contiguous()[:t.shape[0]]


def _short_index_pool(csa, dp):
    """The pool as declared, its tensors followed by two spare pages."""
    return csa.IndexPool(_spare(dp.data), _spare(dp.scale), dp.fmt, dp.dim, dp.page_size)


def _short_kv_pool(csa, dp):
    return csa.KvPool(_spare(dp.latent), _spare(dp.scale), _spare(dp.rope), dp.fmt, dp.page_size)


def _indexer_case(csa):
    g = gen.rng(1500)
    lens = [3000, 700, 64 * 5]
    T = len(lens)
    pt, pool, _ = _index_case(g, "fp8", T, lens)
    qraw = gen.normal(g, (T, 64, 128))
    qcodes, qsc = O.index_prep(qraw, True, "fp8")
    w = gen.uniform(g, (T, 64))
    dpool = _short_index_pool(csa, index_pool_to_device(pool, 64, 128))
    return pt, dpool, t_dev(qcodes), t_dev(qsc.astype(np.float32)), t_dev(w), lens


def test_debug_flag_round_trip(csa):
    assert csa.csa_debug_enabled()
    csa.csa_set_debug(False)
    assert not csa.csa_debug_enabled()
    csa.csa_set_debug(True)
    assert csa.csa_debug_enabled()


def test_debug_valid_calls_unchanged(csa):
    """With debug on, valid calls give the results of debug off."""
    pt, dpool, q, qs, w, lens = _indexer_case(csa)
    T, maxn = len(lens), max(lens)
    # the planted-violation tests need spare pages; here every id is in range
    assert pt.max() < dpool.num_pages
    rs, rl, dpt = t_dev(np.arange(T, dtype=np.int32)), t_dev(np.array(lens, np.int32)), t_dev(pt)
    out = []
    for dbg in (True, False):
        csa.csa_set_debug(dbg)
        logits = torch.full((T, maxn), float("nan"), device=DEV)
        csa.indexer_score(q, w, rs, rl, maxn, dpt, dpool, logits, q_fmt=csa.CSA_FP8_E4M3, q_scale=qs)
        phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
        csa.indexer_topk512(q, w, rs, rl, maxn, dpt, dpool, phys, q_fmt=csa.CSA_FP8_E4M3, q_scale=qs)
        torch.cuda.synchronize()
        out.append((logits.cpu().numpy(), phys.cpu().numpy()))
    csa.csa_set_debug(True)
    np.testing.assert_array_equal(out[0][0], out[1][0])
    np.testing.assert_array_equal(out[0][1], out[1][1])


def _expect_bounds(csa, fn):
    with pytest.raises(csa.CsaError) as e:
        fn()
    assert e.value.status == csa.CSA_ERR_BOUNDS


def test_debug_indexer_bad_page_and_length(csa):
    pt, dpool, q, qs, w, lens = _indexer_case(csa)
    T, maxn = len(lens), max(lens)
    rs, rl = t_dev(np.arange(T, dtype=np.int32)), t_dev(np.array(lens, np.int32))
    bad = pt.copy()
    bad[1, 3] = dpool.num_pages  # a page past the declared pool (inside the tensor)
    logits = torch.full((T + 2, maxn), float("nan"), device=DEV)
    _expect_bounds(csa, lambda: csa.indexer_score(q, w, rs, rl, maxn, t_dev(bad), dpool, logits,
                                                  q_fmt=csa.CSA_FP8_E4M3, q_scale=qs))
    phys = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    _expect_bounds(csa, lambda: csa.indexer_topk512(q, w, rs, rl, maxn, t_dev(bad), dpool, phys,
                                                    q_fmt=csa.CSA_FP8_E4M3, q_scale=qs))
    # a row longer than max_row_len (the table row still covers it)
    long = np.array(lens, np.int32)
    long[2] = 64 * 5 + 3
    _expect_bounds(csa, lambda: csa.indexer_score(q, w, rs, t_dev(long), 64 * 5, t_dev(pt), dpool,
                                                  logits, q_fmt=csa.CSA_FP8_E4M3, q_scale=qs))
    # a negative sequence index
    neg = np.arange(T, dtype=np.int32)
    neg[0] = -1
    _expect_bounds(csa, lambda: csa.indexer_score(q, w, t_dev(neg), rl, maxn, t_dev(pt), dpool,
                                                  logits, q_fmt=csa.CSA_FP8_E4M3, q_scale=qs))
    torch.cuda.synchronize()
    assert torch.isnan(logits).all(), "a rejected call wrote logits"
    assert (phys == -7).all(), "a rejected call wrote a selection"


def test_debug_attention_bad_slot_and_window(csa):
    g = gen.rng(1501)
    Ls = [5000, 700]
    B, H = len(Ls), 16
    pt, c4, raw = _attn_case(g, "fp8", B, Ls, H)
    dc4 = _short_kv_pool(csa, kv_pool_to_device(c4, 64))
    draw = _short_kv_pool(csa, kv_pool_to_device(raw, 256))
    assert pt.max() < draw.num_pages
    sel = np.full((B, 512), -1, np.int32)
    for t, L in enumerate(Ls):
        n = L // 4
        sel[t] = O.topk_page_select(g.standard_normal(n), n, pt[t])[0]
    q, _ = _bf16(gen.normal(g, (B, H, 576)))
    out = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device=DEV)
    qs_, qp = t_dev(np.arange(B, dtype=np.int32)), t_dev(np.array(Ls, np.int32) - 1)
    scale = 576 ** -0.5
    bad = sel.copy()
    bad[1, 5] = dc4.num_pages * 64 + 3  # a slot in the undeclared pages
    _expect_bounds(csa, lambda: csa.csa_sparse_attn(q, qs_, qp, t_dev(bad), dc4, draw, t_dev(pt),
                                                    128, scale, out))
    badw = pt.copy()
    badw[0, (Ls[0] - 1) // 256] = draw.num_pages + 1  # the window's page
    _expect_bounds(csa, lambda: csa.csa_sparse_attn(q, qs_, qp, t_dev(sel), dc4, draw, t_dev(badw),
                                                    128, scale, out))
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all(), "a rejected call wrote its output"
    # the valid call goes through
    csa.csa_sparse_attn(q, qs_, qp, t_dev(sel), dc4, draw, t_dev(pt), 128, scale, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_debug_compress_bad_page(csa):
    g = gen.rng(1502)
    B, rows, ratio = 2, 64, 4
    pages = 3
    num_pages = B * pages + 2
    pt = gen.page_table(g, B, pages, num_pages)
    pool = _short_kv_pool(csa, csa.alloc_kv_pool(num_pages, 64, csa.CSA_FP8_E4M3))
    before = pool.latent.clone()
    x = torch.from_numpy(gen.normal(g, (B * rows, 576)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    cu = t_dev(np.array([0, rows, 2 * rows], np.int32))
    start = t_dev(np.array([0, 64 * 4], np.int32))  # second sequence: entries 64..79, page 1
    gw, gb = torch.zeros(576, device=DEV), torch.zeros(ratio, device=DEV)
    bad = pt.copy()
    bad[1, 1] = pool.num_pages + 1  # the second spare page
    _expect_bounds(csa, lambda: csa.c4_compress(x, cu, start, rows, ratio, gw, gb, t_dev(bad), pool))
    torch.cuda.synchronize()
    assert torch.equal(pool.latent, before), "a rejected call wrote the pool"
    csa.c4_compress(x, cu, start, rows, ratio, gw, gb, t_dev(pt), pool)
    torch.cuda.synchronize()
    assert not torch.equal(pool.latent, before)
