"""indexer_topk512_noalloc (the library's own device scratch, no workspace)
against indexer_topk512 with a caller's workspace: the same kernels, so the
selections must be equal bit for bit. Two calls in a row, the second with a
smaller input (the scratch keeps the first call's contents), then a call that
takes the two-call path (rows grouped by sequence: logits and the top-512
workspace in the scratch), then a call too large for the scratch, which must
be refused before any launch."""
import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests.gpu_helpers import DEV, index_pool_to_device, t_dev
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_c4_amd as m
    return m


def _case(g, fmt, lens, pages_extra=3):
    T = len(lens)
    pps = max((max(n, 1) + 63) // 64 for n in lens)
    P = T * pps + pages_extra
    pt = gen.page_table(g, T, pps, P)
    kraw = gen.normal(g, (P * 64, 128))
    data, sc = O.index_prep(kraw, True, fmt)
    pool = index_pool_to_device(O.IndexPool(data, sc, fmt), 64, 128)
    qc, qs = O.index_prep(gen.normal(g, (T, 64, 128)), True, fmt)
    w = gen.uniform(g, (T, 64))
    qsd = t_dev(qs.astype(np.float32)) if fmt == "fp8" else t_dev(qs)
    return pt, pool, t_dev(qc), qsd, t_dev(w)


def _both(csa, fmt, lens, prep=0, row_seq=None):
    g = gen.rng(4242 + len(lens) + sum(lens) % 1000)
    pt, pool, qc, qs, w = _case(g, fmt, lens)
    T = len(lens)
    rs = t_dev(np.arange(T, dtype=np.int32) if row_seq is None else row_seq)
    rl = t_dev(np.array(lens, np.int32))
    qfmt = csa.CSA_FP8_E4M3 if fmt == "fp8" else csa.CSA_MXFP4
    maxn = max(lens)
    ph_a = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    lg_a = torch.full((T, 512), -7, dtype=torch.int32, device=DEV)
    csa.indexer_topk512_noalloc(qc, w, rs, rl, maxn, t_dev(pt), pool, ph_a, lg_a, q_fmt=qfmt,
                                q_scale=qs, prep=prep)
    ph_b = torch.full((T, 512), -9, dtype=torch.int32, device=DEV)
    lg_b = torch.full((T, 512), -9, dtype=torch.int32, device=DEV)
    csa.indexer_topk512(qc, w, rs, rl, maxn, t_dev(pt), pool, ph_b, lg_b, q_fmt=qfmt, q_scale=qs,
                        prep=prep)
    torch.cuda.synchronize()
    assert torch.equal(ph_a, ph_b), "physical slots differ"
    assert torch.equal(lg_a, lg_b), "logical indices differ"
    # and the result is a valid selection: ascending, -1 tails
    lg = lg_a.cpu().numpy()
    for t, n in enumerate(lens):
        k = min(512, n)
        assert np.all(np.diff(lg[t, :k]) > 0) and np.all(lg[t, k:] == -1)


def test_noalloc_two_calls_then_smaller(csa):
    _both(csa, "fp8", [32768] * 8 + [20000 - 37 * i for i in range(8)])  # fused path, merge lists
    _both(csa, "fp8", [3000, 700, 5, 0, 1500])                          # smaller, on the same scratch


def test_noalloc_mxfp4_and_two_call_path(csa):
    _both(csa, "mxfp4", [150000, 70000])                                 # long rows: merge lists
    q_len = 4
    lens = [9000 - i for i in range(q_len)] + [4000 - i for i in range(q_len)]
    rs = np.repeat(np.arange(2, dtype=np.int32), q_len)
    # rows grouped by sequence: the row-block kernel writes logits into the scratch
    _both(csa, "fp8", lens, prep=csa.CSA_ROWS_PER_SEQ(q_len), row_seq=rs)
    _both(csa, "fp8", [600, 513])


def test_noalloc_refuses_oversized_calls(csa):
    """4096 rows x 33792 entries needs ~0.6 GB of workspace: refused on the
    host, nothing launched, the outputs untouched."""
    T, n = 4096, 33792
    need = csa.csa_workspace_size(csa.CSA_OP_INDEXER_TOPK, T, n, 64)
    assert need > csa.CSA_NOALLOC_SCRATCH_BYTES
    pool = csa.alloc_index_pool(n // 64 + 1, 64, 128, csa.CSA_FP8_E4M3)
    qc = torch.zeros((T, 64, 128), dtype=torch.uint8, device=DEV)
    qs = torch.ones((T, 64), dtype=torch.float32, device=DEV)
    w = torch.ones((T, 64), dtype=torch.float32, device=DEV)
    rs = torch.zeros(T, dtype=torch.int32, device=DEV)
    rl = torch.full((T,), n, dtype=torch.int32, device=DEV)
    pt = t_dev(np.arange(n // 64 + 1, dtype=np.int32)[None])
    ph = torch.full((T, 512), -5, dtype=torch.int32, device=DEV)
    with pytest.raises(csa.CsaError) as e:
        csa.indexer_topk512_noalloc(qc, w, rs, rl, n, pt, pool, ph, q_fmt=csa.CSA_FP8_E4M3, q_scale=qs)
    assert e.value.status == csa.CSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(ph == -5)
