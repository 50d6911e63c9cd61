"""Full-size parity: the benchmark workloads at their real sizes, run through
the library exactly as bench.py runs them (same entry points, same shapes and
so the same launch configurations; the 128K decode also as a HIP-graph
replay), checked on sampled sequences / query rows against the oracle, which
rebuilds those rows from the same seeded draws (tests/fullsize.py).

Bars (as in the small parity tests): logits within 1e-4 of the row's largest
|logit|, plus, per entry, what the few index-K / query codes whose exact value
lies within the float32 evaluation band of a rounding midpoint can change
(tests/quant_band.py); the top-512 equal to the oracle's outside the band of
entries whose logit is within that tolerance of the 512-th largest; attention
(bf16 out) within 2e-2 absolute of the oracle's attention over the entries the
GPU selected, on every sampled row; the step's freshly compressed KV entry /
index-K row checked directly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from tests import fullsize as F
from tests import quant_band as Q

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-4
ATTN_TOL = 2e-2


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_sparse_attention_c4_amd as m
    return m


def _check_csa_row(st: F.SeqState, g_logits, g_phys, pt_row, g_out, label):
    """Logits, selection and attention of one row against the oracle."""
    o_logits, slack = st.scores()
    n = st.row_len
    tol = LOGIT_TOL * np.abs(o_logits).max() + slack
    err = np.abs(g_logits[:n] - o_logits)
    worst = int(np.argmax(err - tol))
    assert np.all(err <= tol), f"{label}: logit {worst} differs by {err[worst]} (tol {tol[worst]})"
    g_log = F.logical_of_phys(g_phys, pt_row)
    ok, equal, nband = F.topk_agrees(o_logits, g_log, 512, tol)
    assert ok, f"{label}: top-512 differs outside the near-tie band ({nband} in band)"
    want = st.attend(g_log[g_log >= 0])
    aerr = np.abs(g_out - want).max()
    assert aerr <= ATTN_TOL, f"{label}: attention differs by {aerr}"
    return equal


def _check_step_writes(W, b, label):
    """The step's compressed entry N-1 and its index-K row, from the pools."""
    L, N = int(W.lens[b]), int(W.N[b])
    slot = int(O.page_slot(W.pt_host[b], N - 1, 64))
    x_new = F.host(W.x_new).reshape(W.B, 4, 576)[b]
    c = O.compress_blocks(x_new, L - 4, 4, F.host(W.gate_w), F.host(W.gate_b))
    cerr = Q.compress_error_bound(x_new, F.host(W.gate_w))
    kv = W.c4_pools[0]
    lat = kv.latent.view(-1, 512)[slot].cpu().numpy()[None]
    sc = kv.scale.view(-1)[slot:slot + 1].cpu().numpy()
    ok, msg, _ = Q.fp8_rows_match(lat, sc, c[:, :512], cerr[None, :512])
    assert ok, f"{label}: compressed latent: {msg}"
    rope = kv.rope.view(-1, 64)[slot].cpu().view(torch.int16).numpy().view(np.uint16)
    ok, msg = Q.bf16_match(rope, c[0, 512:], cerr[512:])
    assert ok, f"{label}: compressed RoPE dims: {msg}"
    k = F.host(W.k_new)[b:b + 1]
    rope = None
    if W.wl.rope_dim:  # the block's index-K row is rotated at the completing token's position
        cos, sin = F.rope_cs([L - 1], W.wl.rope_dim)
        rope = (cos, sin, W.wl.rope_dim)
    ke = Q.exact_rotated(k, W.wl.hadamard, rope=rope)
    kerr = Q.rotation_error_bound(k, W.wl.index_dim, rope=bool(W.wl.rope_dim))
    idx = W.index_pools[0]
    g_codes = idx.data.view(-1, idx.data.shape[-1])[slot].cpu().numpy()[None]
    g_scale = idx.scale.view(idx.data.view(-1, idx.data.shape[-1]).shape[0], -1)[slot].cpu().numpy()
    if W.wl.index_fmt == "fp8":
        ok, msg, _ = Q.fp8_rows_match(g_codes, g_scale.view(np.float32), ke, kerr)
    else:
        ok, msg, _ = Q.mxfp4_rows_match(g_codes, g_scale[None], ke, kerr)
    assert ok, f"{label}: index-K row: {msg}"


def _scan_logits(csa, W):
    """The logits of the step's scan (indexer_score over the same prepared
    queries and pools), after checking that the step's selection is exactly
    their top-512 (topk512_page_select): the step selects on chip without
    writing the logits."""
    W.score_only(0)
    sel = torch.empty_like(W.phys)
    csa.topk512_page_select(W.logits, W.row_len, W.row_seq, W.pt, sel)
    torch.cuda.synchronize()
    assert torch.equal(sel, W.phys), "the step's selection is not the top-512 of its scan's logits"
    return W.logits.cpu().numpy()


def test_decode_128k_sampled(csa):
    """32 x 128K decode (fp8 index-K, 64 + 64 heads): eager step, then the same
    step replayed from a HIP graph must reproduce it bit for bit."""
    from workloads import specs
    from workloads.device import CsaDecode
    wl = specs.DECODE_128K
    W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=1, pool_pages=wl.pool_pages)
    assert W.scan_plan()[0], "the 128K step is expected to select on chip"
    W.step(0)
    torch.cuda.synchronize()
    phys, out = W.phys.clone(), W.out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        W.step(0)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        W.step(0)
    for _ in range(2):
        W.phys.fill_(-7)
        W.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(W.phys, phys)
        assert torch.equal(W.out.view(torch.int16), out.view(torch.int16))
    gl = _scan_logits(csa, W)
    gp, go = phys.cpu().numpy(), out.float().cpu().numpy()
    for b in (0, 4, 9, 13, 18, 22, 27, 31):
        _check_step_writes(W, b, f"seq {b}")
        st = F.decode_seq(W, b)
        _check_csa_row(st, gl[b], gp[b], W.pt_host[b], go[b], f"seq {b}")


def test_spec_decode_128k_sampled(csa):
    """32 x 128K multi-token decode (4 query rows per sequence, the indexer's
    rows-per-sequence hint): the step's selection is the top-512 of its
    scan's logits; sampled rows (causal row lengths N-1 and N, windows ending
    at their own positions) against the oracle."""
    from workloads import specs
    from workloads.device import CsaSpecDecode
    wl = specs.SPEC_DECODE_128K
    W = CsaSpecDecode(wl, [wl.seq_len] * wl.batch, copies=1, pool_pages=wl.pool_pages)
    W.step(0)
    torch.cuda.synchronize()
    gp, go = W.phys.cpu().numpy(), W.out.float().cpu().numpy()
    gl = _scan_logits(csa, W)
    for t in (0, 3, 21, 54, 66, 91, 110, 127):
        st = F.spec_decode_row(W, t)
        b = t // wl.q_len
        _check_csa_row(st, gl[t], gp[t], W.pt_host[b], go[t], f"row {t}")


def test_decode_1m_sampled(csa):
    """4 x 1M decode (MXFP4 index-K, 128 attention heads)."""
    from workloads import specs
    from workloads.device import CsaDecode
    wl = specs.DECODE_1M
    W = CsaDecode(wl, [wl.seq_len] * wl.batch, copies=1, pool_pages=wl.pool_pages)
    W.step(0)
    torch.cuda.synchronize()
    gp, go = W.phys.cpu().numpy(), W.out.float().cpu().numpy()
    gl = _scan_logits(csa, W)
    for b in range(W.B):
        if b in (0, 3):
            _check_step_writes(W, b, f"seq {b}")
        st = F.decode_seq(W, b)
        _check_csa_row(st, gl[b], gp[b], W.pt_host[b], go[b], f"seq {b}")


def test_prefill_4096_on_128k_sampled(csa):
    """Chunked prefill: 4096 new tokens on a 131072-token context, causal
    indexer rows; sampled rows at the start, middle and end of the chunk."""
    from workloads import specs
    from workloads.device import CsaPrefill
    W = CsaPrefill(specs.PREFILL_4K)
    W.step(0)
    torch.cuda.synchronize()
    logits = _scan_logits(csa, W)
    for t in (0, 1, 2, 3, 1709, 2048, 3001, 4095):
        st = F.prefill_row(W, t)
        gl = logits[t]
        gp, go = W.phys[t].cpu().numpy(), W.out[t].float().cpu().numpy()
        _check_csa_row(st, gl, gp, W.pt_host[0], go, f"row {t}")
        n = st.row_len
        assert np.all(np.isfinite(gl[:n]))


def test_hca_csa_ragged_sampled(csa):
    """16 ragged sequences (8K..1M tokens): HCA dense attention of every
    sampled sequence, and the CSA layer of the same step."""
    from workloads import specs
    from workloads.device import HcaCsaRagged
    Wh = HcaCsaRagged(specs.HCA_RAGGED, copies=1)
    Wh.step(0)
    torch.cuda.synchronize()
    ho = Wh.out_hca.float().cpu().numpy()
    W = Wh.csa
    gp, go = W.phys.cpu().numpy(), W.out.float().cpu().numpy()
    gl = _scan_logits(csa, W)
    order = np.argsort(Wh.lens)
    for b in range(Wh.B):
        want = F.hca_oracle(Wh, b)
        err = np.abs(ho[b] - want).max()
        assert err <= ATTN_TOL, f"HCA seq {b} (L={Wh.lens[b]}): differs by {err}"
    for b in (int(order[0]), int(order[3]), int(order[7]), int(order[11]), int(order[-1])):
        st = F.decode_seq(W, b)
        _check_csa_row(st, gl[b], gp[b], W.pt_host[b], go[b], f"CSA seq {b}")
