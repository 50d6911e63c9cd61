"""ctypes declarations of include/csa.h and argument marshalling from torch."""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python compressed_sparse_attention_c4_amd/build.py` "
        "(hipcc, gfx950). There is no fallback implementation.")
lib = C.CDLL(LIB_PATH)

# ---- constants (mirror include/csa.h)
CSA_OK, CSA_ERR_INVALID, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_HIP = range(5)
CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_MXFP4 = range(4)
CSA_PREP_HADAMARD, CSA_PREP_QUANT = 1, 2


def CSA_ROWS_PER_SEQ(n: int) -> int:
    """The rows-per-sequence hint bits of an indexer call's `prep` flags."""
    return (int(n) & 0xFF) << 8
CSA_OP_INDEXER, CSA_OP_TOPK, CSA_OP_CSA_ATTN, CSA_OP_HCA_ATTN, CSA_OP_INDEXER_TOPK = range(5)
CSA_TOPK, CSA_C4_RATIO, CSA_HCA_RATIO, CSA_RAW_PAGE, CSA_C4_PAGE = 512, 4, 128, 256, 64


class _KvPoolC(C.Structure):
    _fields_ = [("latent", C.c_void_p), ("latent_scale", C.c_void_p), ("rope", C.c_void_p),
                ("fmt", C.c_int32), ("page_size", C.c_int32), ("num_pages", C.c_int64)]


class _IndexPoolC(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scale", C.c_void_p), ("fmt", C.c_int32),
                ("dim", C.c_int32), ("page_size", C.c_int32), ("num_pages", C.c_int64)]


_vp, _i32, _i64, _u32, _f32, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_float, C.c_size_t


def _decl(name, args, res=C.c_int):
    f = getattr(lib, name)
    f.argtypes = args
    f.restype = res
    return f


_c4_compress = _decl("c4_compress", [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _KvPoolC, _vp])
_csa_index_prep = _decl("csa_index_prep", [_vp, _i32, _i64, _i32, _u32, _i32, _vp, _vp, _vp, _vp])
_decode_prep = _decl("csa_decode_prep", [_vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _i32, _KvPoolC,
                                         _vp, _i32, _KvPoolC, _vp, _vp, _i32, _i32, _u32,
                                         _IndexPoolC, _vp, _vp, _vp])
_indexer_score = _decl("indexer_score", [_vp, _i32, _vp, _u32, _vp, _i32, _i32, _i32, _vp, _vp, _i32,
                                         _vp, _i32, _IndexPoolC, _vp, _i64, _vp, _vp, _vp, _sz, _vp])
_indexer_topk = _decl("indexer_topk512", [_vp, _i32, _vp, _u32, _vp, _i32, _i32, _i32, _vp, _vp, _i32,
                                          _vp, _i32, _IndexPoolC, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
                                          _vp])
_topk = _decl("topk512_page_select", [_vp, _i64, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp])
_csa_attn = _decl("csa_sparse_attn", [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _KvPoolC, _KvPoolC,
                                      _vp, _i32, _i32, _f32, _vp, _i32, _vp, _sz, _vp])
_hca_attn = _decl("hca_dense_attn", [_vp, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _KvPoolC, _vp, _i32,
                                     _KvPoolC, _vp, _i32, _i32, _f32, _vp, _i32, _vp, _sz, _vp])
_ws_size = _decl("csa_workspace_size", [_i32, _i64, _i64, _i32], _sz)
_status_string = _decl("csa_status_string", [C.c_int], C.c_char_p)
_version = _decl("csa_version", [], C.c_char_p)


class CsaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {csa_status_string(status)} (status {status})")
        self.status = status


def csa_status_string(status: int) -> str:
    return _status_string(status).decode()


def csa_version() -> str:
    return _version().decode()


def csa_workspace_size(op: int, rows: int, max_len: int, heads: int) -> int:
    return int(_ws_size(op, rows, max_len, heads))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _fmt_of(t: torch.Tensor, declared: int | None = None) -> int:
    if declared is not None:
        return declared
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise ValueError(f"cannot infer a csa format from {t.dtype}; pass fmt")


def _check(name, status):
    if status != CSA_OK:
        raise CsaError(name, status)


@dataclass
class KvPool:
    """KV pool tensors: latent [P, ps, 512] (uint8 e4m3 codes or float32),
    scale [P, ps] float32 (FP8 only), rope [P, ps, 64] (bf16 or float32)."""
    latent: torch.Tensor
    scale: torch.Tensor | None
    rope: torch.Tensor
    fmt: int
    page_size: int

    @property
    def num_pages(self) -> int:
        return self.latent.shape[0]

    def c(self) -> _KvPoolC:
        return _KvPoolC(_ptr(self.latent), _ptr(self.scale), _ptr(self.rope), self.fmt,
                        self.page_size, self.num_pages)


@dataclass
class IndexPool:
    """Index-K pool tensors: data [P, ps, dim | dim/2], scale [P, ps] float32
    (FP8) or [P, ps, dim/32] uint8 (MXFP4) or None (F32)."""
    data: torch.Tensor
    scale: torch.Tensor | None
    fmt: int
    dim: int
    page_size: int

    @property
    def num_pages(self) -> int:
        return self.data.shape[0]

    def c(self) -> _IndexPoolC:
        return _IndexPoolC(_ptr(self.data), _ptr(self.scale), self.fmt, self.dim, self.page_size,
                           self.num_pages)


def c4_compress(x, cu_rows, start_pos, max_rows, ratio, gate_w, gate_b, page_table, out: KvPool,
                stream=None):
    B = cu_rows.numel() - 1
    _check("c4_compress", _c4_compress(
        _ptr(x), _fmt_of(x), _ptr(cu_rows), _ptr(start_pos), B, int(max_rows), int(ratio),
        _ptr(gate_w), _ptr(gate_b), _ptr(page_table), page_table.shape[-1], out.c(),
        _stream(stream)))


def csa_index_prep(v, dim, flags, out_fmt, out, out_scale=None, dst_rows=None, stream=None):
    rows = v.numel() // dim
    _check("csa_index_prep", _csa_index_prep(
        _ptr(v), _fmt_of(v), rows, int(dim), int(flags), int(out_fmt), _ptr(out), _ptr(out_scale),
        _ptr(dst_rows), _stream(stream)))


def csa_decode_prep(x, pos, gate_w, gate_b, page_table, c4: KvPool, raw_page_table, raw: KvPool,
                    k_rows=None, q_rows=None, kpool: IndexPool | None = None, q_out=None,
                    q_out_scale=None, flags=CSA_PREP_HADAMARD, stream=None):
    """x [B][ratio][576]; pos int32 [B]; k_rows [B][dim], q_rows [B][H_I][dim] (bf16 or f32)."""
    B, ratio = x.shape[0], x.shape[1]
    kq = k_rows if k_rows is not None else q_rows
    H_I = q_rows.shape[1] if q_rows is not None else 0
    kp = kpool.c() if kpool is not None else _IndexPoolC(None, None, CSA_F32, 128, c4.page_size, 0)
    _check("csa_decode_prep", _decode_prep(
        _ptr(x), _fmt_of(x), _ptr(pos), B, ratio, _ptr(gate_w), _ptr(gate_b), _ptr(page_table),
        page_table.shape[-1], c4.c(), _ptr(raw_page_table), raw_page_table.shape[-1], raw.c(),
        _ptr(k_rows), _ptr(q_rows), _fmt_of(kq) if kq is not None else CSA_BF16, H_I, int(flags),
        kp, _ptr(q_out), _ptr(q_out_scale), _stream(stream)))


def indexer_score(q, w, row_seq, row_len, max_row_len, page_table, k: IndexPool, logits, *,
                  q_fmt=None, q_scale=None, prep=0, q_used=None, q_used_scale=None, ws=None,
                  stream=None):
    T, H_I = w.shape
    D_I = k.dim
    if ws is None and prep & CSA_PREP_QUANT and q_used is None:
        n = csa_workspace_size(CSA_OP_INDEXER, T, max_row_len, H_I)
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check("indexer_score", _indexer_score(
        _ptr(q), _fmt_of(q, q_fmt), _ptr(q_scale), int(prep), _ptr(w), T, H_I, D_I, _ptr(row_seq),
        _ptr(row_len), int(max_row_len), _ptr(page_table), page_table.shape[-1], k.c(),
        _ptr(logits), logits.shape[-1], _ptr(q_used), _ptr(q_used_scale), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))


def indexer_topk512(q, w, row_seq, row_len, max_row_len, page_table, k: IndexPool, phys_idx,
                    logical_idx=None, *, q_fmt=None, q_scale=None, prep=0, q_used=None,
                    q_used_scale=None, ws=None, scan_done=None, stream=None):
    """scan_done: optional torch.cuda.Event, recorded right after the scan launch."""
    T, H_I = w.shape
    if ws is None:
        n = csa_workspace_size(CSA_OP_INDEXER_TOPK, T, max_row_len, H_I)
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    ev = None
    if scan_done is not None:
        # the handle exists after a first record; recording it here, in front
        # of the scan, costs a few microseconds of stream time, so a caller
        # that times the scan records its events once beforehand
        if not scan_done.cuda_event:
            scan_done.record()
        ev = scan_done.cuda_event
    _check("indexer_topk512", _indexer_topk(
        _ptr(q), _fmt_of(q, q_fmt), _ptr(q_scale), int(prep), _ptr(w), T, H_I, k.dim, _ptr(row_seq),
        _ptr(row_len), int(max_row_len), _ptr(page_table), page_table.shape[-1], k.c(),
        _ptr(phys_idx), _ptr(logical_idx), _ptr(q_used), _ptr(q_used_scale), _ptr(ws),
        ws.numel(), ev, _stream(stream)))


def topk512_page_select(logits, row_len, row_seq, page_table, phys_idx, logical_idx=None,
                        c4_page_size=CSA_C4_PAGE, ws=None, stream=None):
    R = row_len.numel()
    ld = logits.shape[-1]
    if ws is None:
        n = csa_workspace_size(CSA_OP_TOPK, R, ld, 1)
        ws = torch.empty(n, dtype=torch.uint8, device=logits.device) if n else None
    _check("topk512_page_select", _topk(
        _ptr(logits), ld, R, _ptr(row_len), _ptr(row_seq), _ptr(page_table),
        page_table.shape[-1], int(c4_page_size), _ptr(phys_idx), _ptr(logical_idx), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))


def _attn_ws(op, T, entries, H, device, ws):
    if ws is not None:
        return ws
    n = csa_workspace_size(op, T, entries, H)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def csa_sparse_attn(q, q_seq, q_pos, phys_idx, c4: KvPool, raw: KvPool, raw_page_table, window,
                    softmax_scale, out, ws=None, stream=None):
    T, H = q.shape[0], q.shape[1]
    k_sel = phys_idx.shape[-1]
    ws = _attn_ws(CSA_OP_CSA_ATTN, T, k_sel + window, H, q.device, ws)
    _check("csa_sparse_attn", _csa_attn(
        _ptr(q), _fmt_of(q), T, H, _ptr(q_seq), _ptr(q_pos), _ptr(phys_idx), k_sel, c4.c(), raw.c(),
        _ptr(raw_page_table), raw_page_table.shape[-1], int(window), float(softmax_scale),
        _ptr(out), _fmt_of(out), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def hca_dense_attn(q, q_seq, q_pos, max_len, ratio, hca: KvPool, hca_page_table, raw: KvPool,
                   raw_page_table, window, softmax_scale, out, ws=None, stream=None):
    T, H = q.shape[0], q.shape[1]
    ws = _attn_ws(CSA_OP_HCA_ATTN, T, max_len // ratio + window, H, q.device, ws)
    _check("hca_dense_attn", _hca_attn(
        _ptr(q), _fmt_of(q), T, H, _ptr(q_seq), _ptr(q_pos), int(max_len), int(ratio), hca.c(),
        _ptr(hca_page_table), hca_page_table.shape[-1], raw.c(), _ptr(raw_page_table),
        raw_page_table.shape[-1], int(window), float(softmax_scale), _ptr(out), _fmt_of(out),
        _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
