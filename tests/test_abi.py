"""CPU checks of the C ABI: libcsa.so loads, exports every function that
include/csa.h declares, and rejects bad arguments on the host before any
launch (no GPU call is made on these paths)."""
import ctypes as C
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "csa.h")
LIB = os.path.join(ROOT, "compressed_sparse_attention_c4_amd", "libcsa.so")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:csa_status|size_t|const char\s*\*|char\s*\*)\s*\**\s*(\w+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libcsa.so not built")
    return C.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("c4_compress", "csa_index_prep", "csa_decode_prep", "indexer_score", "topk512_page_select",
              "csa_sparse_attn", "hca_dense_attn", "csa_workspace_size", "csa_status_string",
              "csa_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in csa.h but not exported"


class KvPoolC(C.Structure):
    _fields_ = [("latent", C.c_void_p), ("latent_scale", C.c_void_p), ("rope", C.c_void_p),
                ("fmt", C.c_int32), ("page_size", C.c_int32), ("num_pages", C.c_int64)]


class RopeC(C.Structure):
    _fields_ = [("pos", C.c_void_p), ("cos_sin", C.c_void_p), ("dim", C.c_int32),
                ("rows_per_pos", C.c_int32)]


NO_ROPE = RopeC(None, None, 0, 1)


class IndexPoolC(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scale", C.c_void_p), ("fmt", C.c_int32),
                ("dim", C.c_int32), ("page_size", C.c_int32), ("num_pages", C.c_int64)]


INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
FAKE = 0x1000  # never dereferenced: every call below fails its host checks


def test_status_strings_and_version(lib):
    lib.csa_status_string.restype = C.c_char_p
    lib.csa_version.restype = C.c_char_p
    assert lib.csa_status_string(0) == b"ok"
    assert lib.csa_status_string(1) == b"invalid argument"
    assert lib.csa_version().count(b".") == 2
    assert b"debug" in lib.csa_status_string(5)


def test_debug_mode_switch(lib):
    """csa_set_debug / csa_debug_enabled are host state only; the mode starts
    from CSA_DEBUG (unset here)."""
    lib.csa_debug_enabled.restype = C.c_int32
    lib.csa_set_debug.argtypes = [C.c_int32]
    start = lib.csa_debug_enabled()
    try:
        lib.csa_set_debug(1)
        assert lib.csa_debug_enabled() == 1
        lib.csa_set_debug(0)
        assert lib.csa_debug_enabled() == 0
    finally:
        lib.csa_set_debug(start)


def test_workspace_sizes(lib):
    lib.csa_workspace_size.restype = C.c_size_t
    lib.csa_workspace_size.argtypes = [C.c_int32, C.c_int64, C.c_int64, C.c_int32]
    assert lib.csa_workspace_size(1, 128, 16384, 1) == 0          # one launch per row
    assert lib.csa_workspace_size(1, 128, 32768, 1) == 128 * 2 * 512 * 8  # two 16384-key chunks
    assert lib.csa_workspace_size(1, 4096, 33792, 1) == 4096 * 9 * 512 * 8  # nine 4096-key chunks
    assert lib.csa_workspace_size(1, 32, 32768, 1) >= 32 * 512 * 8  # chunk candidates
    assert lib.csa_workspace_size(1, 4, 1 << 20, 1) >= 4 * 512 * 8
    assert lib.csa_workspace_size(0, 32, 0, 64) >= 32 * 64 * 132  # prepared query
    assert lib.csa_workspace_size(2, -1, 10, 64) == 0
    # indexer + top-512: the query area, then candidates (or logits and the
    # top-512 workspace), whichever is larger
    assert lib.csa_workspace_size(4, 32, 32768, 64) >= 32 * 32768 * 4
    assert lib.csa_workspace_size(4, 4, 262144, 64) >= 4 * 64 * 512 * 12


def _two_phase_bytes(T, H, e_pad, ch):
    # P' bf16 [T][H][e_pad], chunk statistics float2 [T][H][e_pad / ch], then
    # the entries' slots int32 [T][e_pad] (value copies of 4 MB or more gather)
    up = lambda n: (n + 255) // 256 * 256
    src = up(T * H * e_pad * 2) + up(T * H * (e_pad // ch) * 8)
    copy = T * e_pad * 512
    return src + (T * e_pad * 4 if copy >= 4 << 20 else copy)


def test_decode_attention_chunk_plan(lib):
    """Decode attention's phase A takes 64-entry chunks while their grid fits
    the 256 CUs, else 96-entry chunks when those fit (the workspace size shows
    which: its chunk statistics and padding follow the chunk length)."""
    lib.csa_workspace_size.restype = C.c_size_t
    lib.csa_workspace_size.argtypes = [C.c_int32, C.c_int64, C.c_int64, C.c_int32]
    csa_attn = 2
    # 24 queries x 10 chunks of 64: 240 workgroups
    assert lib.csa_workspace_size(csa_attn, 24, 640, 64) == _two_phase_bytes(24, 64, 640, 64)
    # 32 queries: 320 workgroups of 64 entries, 224 of 96 (7 chunks, 672 padded)
    assert lib.csa_workspace_size(csa_attn, 32, 640, 64) == _two_phase_bytes(32, 64, 672, 96)
    # 48 queries: neither fits one round; 64-entry chunks
    assert lib.csa_workspace_size(csa_attn, 48, 640, 64) == _two_phase_bytes(48, 64, 640, 64)
    # 4 queries x 128 heads (value copy, no gather)
    assert lib.csa_workspace_size(csa_attn, 4, 640, 128) == _two_phase_bytes(4, 128, 640, 64)


def test_compress_rejects_bad_arguments(lib):
    f = lib.c4_compress
    f.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, KvPoolC, C.c_void_p]
    good = KvPoolC(FAKE, FAKE, FAKE, 2, 64, 10)
    assert f(FAKE, 1, FAKE, FAKE, 1, 16, 0, FAKE, FAKE, FAKE, 4, good, None) == INVALID      # ratio 0
    assert f(FAKE, 1, FAKE, FAKE, 1, 16, 2000, FAKE, FAKE, FAKE, 4, good, None) == INVALID   # ratio > 1024
    assert f(FAKE, 3, FAKE, FAKE, 1, 16, 4, FAKE, FAKE, FAKE, 4, good, None) == INVALID      # x fmt MXFP4
    bad_pool = KvPoolC(FAKE, None, FAKE, 2, 64, 10)                                          # FP8 without scale
    assert f(FAKE, 1, FAKE, FAKE, 1, 16, 4, FAKE, FAKE, FAKE, 4, bad_pool, None) == INVALID
    assert f(None, 1, FAKE, FAKE, 1, 16, 4, FAKE, FAKE, FAKE, 4, good, None) == INVALID      # null x
    assert f(FAKE, 1, FAKE, FAKE, 0, 16, 4, FAKE, FAKE, FAKE, 4, good, None) == 0            # B = 0: no-op


def test_decode_prep_rejects_bad_arguments(lib):
    f = lib.csa_decode_prep
    f.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                  C.c_void_p, C.c_int32, KvPoolC, C.c_void_p, C.c_int32, KvPoolC, C.c_void_p,
                  C.c_void_p, C.c_int32, C.c_int32, C.c_uint32, RopeC, IndexPoolC, C.c_void_p,
                  C.c_void_p, C.c_void_p]
    c4 = KvPoolC(FAKE, FAKE, FAKE, 2, 64, 10)
    raw = KvPoolC(FAKE, FAKE, FAKE, 2, 256, 10)
    kp = IndexPoolC(FAKE, FAKE, 2, 128, 64, 10)

    def call(x=FAKE, x_fmt=1, B=2, ratio=4, c4p=c4, rawp=raw, k=FAKE, q=FAKE, kq_fmt=1, H_I=64,
             flags=1, rope=NO_ROPE, kpool=kp, q_out=FAKE, q_sc=FAKE):
        return f(x, x_fmt, FAKE, B, ratio, FAKE, FAKE, FAKE, 8, c4p, FAKE, 4, rawp, k, q, kq_fmt,
                 H_I, flags, rope, kpool, q_out, q_sc, None)

    assert call(ratio=0) == INVALID
    assert call(ratio=129) == INVALID
    assert call(x_fmt=2) == INVALID                                    # x must be bf16 / f32
    assert call(rawp=KvPoolC(FAKE, FAKE, FAKE, 0, 256, 10)) == INVALID  # c4 FP8, raw F32
    assert call(flags=2) == INVALID                                    # Hadamard / rope flags only
    assert call(flags=5) == INVALID                                    # rope without a table
    assert call(flags=5, rope=RopeC(None, FAKE, 63, 1)) == INVALID     # odd rope dim
    assert call(flags=5, rope=RopeC(None, FAKE, 130, 1)) == INVALID    # rope dim > row dim
    assert call(kpool=IndexPoolC(FAKE, FAKE, 2, 96, 64, 10)) == INVALID  # dim 96
    assert call(kpool=IndexPoolC(FAKE, FAKE, 2, 128, 32, 10)) == INVALID  # page size != c4's
    assert call(q_out=None) == INVALID                                 # q rows without an output
    assert call(kq_fmt=2) == INVALID                                   # k / q rows must be raw
    assert call(x=None) == INVALID
    assert call(B=0) == 0                                              # nothing to do


def test_index_prep_rejects_bad_arguments(lib):
    f = lib.csa_index_prep
    f.argtypes = [C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_uint32, C.c_int32, C.c_void_p,
                  C.c_void_p, C.c_void_p, RopeC, C.c_void_p]
    ok_rope = RopeC(FAKE, FAKE, 64, 64)
    assert f(FAKE, 1, 10, 128, 5, 2, FAKE, FAKE, None, NO_ROPE, None) == INVALID     # rope, no table
    assert f(FAKE, 1, 10, 128, 5, 2, FAKE, FAKE, None, RopeC(FAKE, FAKE, 64, 0), None) == INVALID
    assert f(FAKE, 1, 10, 64, 5, 2, FAKE, FAKE, None, RopeC(FAKE, FAKE, 66, 1), None) == INVALID
    assert f(FAKE, 1, 10, 128, 8, 2, FAKE, FAKE, None, ok_rope, None) == INVALID       # unknown flag
    assert f(FAKE, 1, 0, 128, 5, 2, FAKE, FAKE, None, ok_rope, None) == 0              # no rows


def test_indexer_rejects_bad_arguments(lib):
    f = lib.indexer_score
    f.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_uint32, C.c_void_p, C.c_int32, C.c_int32,
                  C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, IndexPoolC,
                  C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    fp8 = IndexPoolC(FAKE, FAKE, 2, 128, 64, 10)
    # raw bf16 query without the quant flag
    assert f(FAKE, 1, None, 1, FAKE, 4, 64, 128, FAKE, FAKE, 100, FAKE, 2, fp8, FAKE, 100, None, None,
             FAKE, 1 << 20, None) == INVALID
    # 32 heads on the MFMA path
    assert f(FAKE, 2, FAKE, 0, FAKE, 4, 32, 128, FAKE, FAKE, 100, FAKE, 2, fp8, FAKE, 100, None, None,
             None, 0, None) == UNSUPPORTED
    # ld smaller than the longest row
    assert f(FAKE, 2, FAKE, 0, FAKE, 4, 64, 128, FAKE, FAKE, 100, FAKE, 2, fp8, FAKE, 99, None, None,
             None, 0, None) == INVALID
    # in-call preparation without workspace or q_used
    assert f(FAKE, 1, None, 3, FAKE, 4, 64, 128, FAKE, FAKE, 100, FAKE, 2, fp8, FAKE, 100, None, None,
             None, 0, None) == WORKSPACE
    # prepared query of the wrong format
    assert f(FAKE, 3, FAKE, 0, FAKE, 4, 64, 128, FAKE, FAKE, 100, FAKE, 2, fp8, FAKE, 100, None, None,
             None, 0, None) == INVALID


def test_indexer_topk512_rejects_bad_arguments(lib):
    f = lib.indexer_topk512
    f.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_uint32, C.c_void_p, C.c_int32, C.c_int32,
                  C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, IndexPoolC,
                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p,
                  C.c_void_p]
    lib.csa_workspace_size.restype = C.c_size_t
    lib.csa_workspace_size.argtypes = [C.c_int32, C.c_int64, C.c_int64, C.c_int32]
    fp8 = IndexPoolC(FAKE, FAKE, 2, 128, 64, 10)
    need = lib.csa_workspace_size(4, 4, 100, 64)

    def call(q_fmt=2, prep=0, H_I=64, max_len=100, pool=fp8, phys=FAKE, ws=FAKE, ws_bytes=None):
        return f(FAKE, q_fmt, FAKE, prep, FAKE, 4, H_I, 128, FAKE, FAKE, max_len, FAKE, 2, pool, phys,
                 None, None, None, ws, need if ws_bytes is None else ws_bytes, None, None)

    assert call(q_fmt=1, prep=1) == INVALID                 # raw bf16 query without the quant flag
    assert call(H_I=32) == UNSUPPORTED                      # 32 heads on the MFMA path
    assert call(q_fmt=3) == INVALID                         # prepared query of the wrong format
    assert call(max_len=1 << 22) == UNSUPPORTED             # longer than the top-512 handles
    assert call(ws=None) == WORKSPACE                       # the workspace is always needed
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(phys=None) == INVALID                       # phys_idx is required
    assert call(max_len=-1) == INVALID
    # the rows-per-sequence hint occupies bits 8..15 of prep; other bits are invalid
    assert call(prep=1 << 16) == INVALID
    assert call(q_fmt=3, prep=4 << 8) == INVALID            # the hint does not mask other errors
    assert call(phys=None, prep=4 << 8) == INVALID           # (checks run before any launch)


def test_topk_and_attention_reject_bad_arguments(lib):
    t = lib.topk512_page_select
    t.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                  C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    assert t(FAKE, 100, 2, FAKE, FAKE, FAKE, 4, 0, FAKE, None, None, 0, None) == INVALID
    assert t(FAKE, 100, 2, FAKE, FAKE, FAKE, 4, 64, None, None, None, 0, None) == INVALID
    assert t(FAKE, 100, 0, FAKE, FAKE, FAKE, 4, 64, FAKE, None, None, 0, None) == 0
    g = lib.topk_page_select
    g.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                  C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    assert g(FAKE, 100, 2, FAKE, FAKE, FAKE, 4, 64, 0, FAKE, None, None, 0, None) == INVALID      # k = 0
    assert g(FAKE, 100, 2, FAKE, FAKE, FAKE, 4, 64, 2049, FAKE, None, None, 0, None) == INVALID   # k > 2048
    assert g(FAKE, 1 << 20, 2, FAKE, FAKE, FAKE, 4, 64, 2048, FAKE, None, None, 0, None) == UNSUPPORTED
    assert g(FAKE, 200000, 2, FAKE, FAKE, FAKE, 4, 64, 2048, FAKE, None, None, 0, None) == WORKSPACE
    a = lib.csa_sparse_attn
    a.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                  C.c_int32, KvPoolC, KvPoolC, C.c_void_p, C.c_int32, C.c_int32, C.c_float,
                  C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]
    fp8 = KvPoolC(FAKE, FAKE, FAKE, 2, 64, 10)
    raw = KvPoolC(FAKE, FAKE, FAKE, 2, 256, 10)
    f32 = KvPoolC(FAKE, None, FAKE, 0, 256, 10)
    assert a(FAKE, 1, 2, 64, FAKE, FAKE, FAKE, 2049, fp8, raw, FAKE, 4, 128, 0.04, FAKE, 1, FAKE, 1 << 30, None) == INVALID
    assert a(FAKE, 1, 2, 64, FAKE, FAKE, FAKE, 512, fp8, f32, FAKE, 4, 128, 0.04, FAKE, 1, FAKE, 1 << 30, None) == INVALID
    assert a(FAKE, 1, 2, 64, FAKE, FAKE, FAKE, 512, fp8, raw, FAKE, 4, -1, 0.04, FAKE, 1, FAKE, 1 << 30, None) == INVALID
    assert a(FAKE, 1, 2, 64, FAKE, FAKE, FAKE, 0, fp8, raw, FAKE, 4, 0, 0.04, FAKE, 1, FAKE, 1 << 30, None) == INVALID
    assert a(FAKE, 1, 2, 48, FAKE, FAKE, FAKE, 512, fp8, raw, FAKE, 4, 128, 0.04, FAKE, 1, FAKE, 1 << 30, None) == UNSUPPORTED
    # two queries over 640 entries are split over several workgroups: needs a workspace
    assert a(FAKE, 1, 2, 64, FAKE, FAKE, FAKE, 512, fp8, raw, FAKE, 4, 128, 0.04, FAKE, 1, None, 0, None) == WORKSPACE


def test_noalloc_refuses_oversized_and_bad_sizes(lib):
    """indexer_topk512_noalloc checks its sizes against its fixed scratch on
    the host before touching the GPU: too large a call is CSA_ERR_WORKSPACE,
    negative sizes CSA_ERR_INVALID."""
    f = lib.indexer_topk512_noalloc
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_uint32, C.c_void_p, C.c_int32, C.c_int32,
                  C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, IndexPoolC,
                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    pool = IndexPoolC(FAKE, FAKE, 2, 128, 64, 1000)
    args = lambda T, n: (FAKE, 2, FAKE, 0, FAKE, T, 64, 128, FAKE, FAKE, n, FAKE, 600, pool, FAKE,
                         None, None, None, None)
    assert f(*args(4096, 33792)) == WORKSPACE
    assert f(*args(-1, 1000)) == INVALID
    assert f(*args(4, -5)) == INVALID


def test_hisparse_rejects_bad_arguments(lib):
    f = lib.hisparse_swap_in
    f.restype = C.c_int
    f.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, KvPoolC, C.c_void_p, C.c_int32, KvPoolC,
                  C.c_int32, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                  C.c_void_p]
    fp8 = KvPoolC(FAKE, FAKE, FAKE, 2, 64, 10)
    f32 = KvPoolC(FAKE, None, FAKE, 0, 64, 10)

    def call(R=2, k=512, hot=1024, far=fp8, near=fp8, step=0, max_entries=1000, sel=FAKE):
        return f(sel, R, k, FAKE, far, FAKE, 4, near, hot, FAKE, max_entries, FAKE, FAKE, step, FAKE, None)

    assert call(k=513) == INVALID           # more than 512 selected entries per row
    assert call(hot=511) == INVALID         # fewer hot slots than selected entries
    assert call(hot=4097) == INVALID
    assert call(near=f32) == INVALID        # far and near formats differ
    assert call(step=-1) == INVALID
    assert call(sel=None) == INVALID
    assert call(R=0) == 0


def test_binding_rejects_short_gate_parameters():
    """The binding checks the gate sizes before calling the library: the
    compressor reads 576 weights and one positional bias per block row, so a
    shorter tensor would be read past its end."""
    if not os.path.exists(LIB):
        pytest.skip("libcsa.so not built")
    import torch
    import compressed_sparse_attention_c4_amd as csa
    x = torch.zeros(8, 576)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    start = torch.zeros(1, dtype=torch.int32)
    pt = torch.zeros(1, 1, dtype=torch.int32)
    pool = csa.KvPool(torch.zeros(1, 64, 512, dtype=torch.uint8), torch.zeros(1, 64),
                      torch.zeros(1, 64, 64, dtype=torch.bfloat16), csa.CSA_FP8_E4M3, 64)
    with pytest.raises(ValueError, match="gate_b"):
        csa.c4_compress(x, cu, start, 8, 4, torch.zeros(576), torch.zeros(1), pt, pool)
    with pytest.raises(ValueError, match="gate_w"):
        csa.c4_compress(x, cu, start, 8, 4, torch.zeros(64), torch.zeros(4), pt, pool)
    with pytest.raises(ValueError, match="gate_b"):
        csa.csa_decode_prep(torch.zeros(2, 4, 576), torch.zeros(2, dtype=torch.int32),
                            torch.zeros(576), torch.zeros(3), pt, pool, pt, pool)


def test_binding_rejects_short_buffers():
    """The binding compares the tensors it passes with the sizes the call
    implies (the library sees only pointers)."""
    if not os.path.exists(LIB):
        pytest.skip("libcsa.so not built")
    import torch
    import compressed_sparse_attention_c4_amd as csa
    T = 4
    q, w = torch.zeros(T, 64, 128), torch.zeros(T, 64)
    rs, rl = torch.zeros(T, dtype=torch.int32), torch.zeros(T, dtype=torch.int32)
    pt = torch.zeros(T, 1, dtype=torch.int32)
    pool = csa.IndexPool(torch.zeros(1, 64, 128, dtype=torch.uint8), torch.zeros(1, 64),
                         csa.CSA_FP8_E4M3, 128, 64)
    with pytest.raises(ValueError, match="phys_idx"):
        csa.indexer_topk512(q, w, rs, rl, 64, pt, pool, torch.zeros(T, 100, dtype=torch.int32))
    with pytest.raises(ValueError, match="row_len"):
        csa.indexer_topk512(q, w, rs, rl[:2], 64, pt, pool, torch.zeros(T, 512, dtype=torch.int32))
    with pytest.raises(ValueError, match="logits"):
        csa.indexer_score(q, w, rs, rl, 64, pt, pool, torch.zeros(T - 1, 64))
    with pytest.raises(ValueError, match="phys_idx"):
        csa.topk_page_select(torch.zeros(T, 64), rl, rs, pt, 8, torch.zeros(T, 4, dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        csa.csa_index_prep(torch.zeros(T, 128), 128, 0, csa.CSA_FP8_E4M3, torch.zeros(T * 64, dtype=torch.uint8),
                           torch.zeros(T))
    kv = csa.KvPool(torch.zeros(1, 64, 512, dtype=torch.uint8), torch.zeros(1, 64),
                    torch.zeros(1, 64, 64, dtype=torch.bfloat16), csa.CSA_FP8_E4M3, 64)
    with pytest.raises(ValueError, match="out"):
        csa.csa_sparse_attn(torch.zeros(T, 64, 576, dtype=torch.bfloat16), rs, rs,
                            torch.zeros(T, 512, dtype=torch.int32), kv, kv, pt, 128, 0.04,
                            torch.zeros(T, 64, 256, dtype=torch.bfloat16))
