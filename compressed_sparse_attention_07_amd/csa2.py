"""Thin Python binding of the CSA2 C ABI (include/csa2.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libcsa2.so.  torch tensors supply device memory and the current stream.  There
is no fallback: if the library is missing, or a tensor is not on the GPU, the
call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_CAPACITY, ERR_LAUNCH, ERR_SCRATCH = range(8)
OP_INDEX_FULL, OP_INDEX_REINDEX, OP_ATTEND = 1, 2, 3
KV_DIM, IDX_DIM, BLOCK = 128, 64, 8
SIZE_MAX = (1 << 64) - 1  # csa2_workspace_bytes: sizes out of range

EXPORTS = (
    "fp4_kv_append",
    "fp8_window_append",
    "csa2_index_full",
    "csa2_index_full_prep",
    "csa2_index_full_scan",
    "csa2_index_full_select",
    "csa2_index_reindex",
    "csa2_index_reindex_noalloc",
    "mxfp4_key_append",
    "csa2_index_full_mx",
    "csa2_index_full_mx_scan",
    "csa2_index_full_scan_timed",
    "csa2_index_reindex_timed",
    "csa2_attend_timed",
    "csa2_stream_read_groups",
    "csa2_stream_read",
    "csa2_index_reindex_mx",
    "csa2_attend",
    "csa2_attend_fp8win",
    "csa2_reindex_attend",
    "csa2_token_append",
    "csa2_window_append",
    "csa2_workspace_bytes",
    "csa2_workspace_init",
    "csa2_status_string",
    "csa2_version",
)


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


class SeqsC(ctypes.Structure):
    _fields_ = [
        ("kv_row0", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p),
        ("n_q", ctypes.c_int32),
        ("max_len_ub", ctypes.c_int32),
        ("total_len_ub", ctypes.c_int64),
        ("cache_rows", ctypes.c_int64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcsa2.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_sparse_attention_07_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        L.fp4_kv_append.argtypes = [vp, i64, i32, vp, i64, vp, vp, i64, vp]
        for name in ("csa2_index_full", "csa2_index_full_prep", "csa2_index_full_scan", "csa2_index_full_select"):
            getattr(L, name).argtypes = [vp, vp, vp, SeqsC, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
            getattr(L, name).restype = ctypes.c_int
        L.csa2_index_reindex.argtypes = [vp, vp, vp, SeqsC, i32, vp, i32, i32, i32, vp, vp, sz, vp]
        L.csa2_index_reindex_noalloc.argtypes = [vp, vp, vp, SeqsC, i32, vp, i32, i32, i32, vp, vp]
        L.csa2_attend.argtypes = [vp, vp, vp, SeqsC, vp, i32, vp, vp, i32, i64, i32, vp, i32, f32, vp, vp, sz, vp]
        L.fp8_window_append.argtypes = [vp, i64, i32, vp, i64, vp, i64, vp]
        L.mxfp4_key_append.argtypes = [vp, i64, i32, vp, i64, vp, vp, i64, vp]
        for name in ("csa2_index_full_mx", "csa2_index_full_mx_scan"):
            getattr(L, name).argtypes = [vp, vp, vp, vp, SeqsC, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
        L.csa2_index_reindex_mx.argtypes = [vp, vp, vp, vp, SeqsC, i32, vp, i32, i32, i32, vp, vp, sz, vp]
        L.csa2_index_full_scan_timed.argtypes = [vp, vp, vp, vp, SeqsC, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp,
                                                 vp, vp]
        L.csa2_attend_fp8win.argtypes = [vp, vp, vp, SeqsC, vp, i32, vp, vp, i32, i64, i32, vp, vp, i32, f32, vp,
                                         vp, sz, vp]
        L.csa2_reindex_attend.argtypes = [vp, vp, vp, vp, SeqsC, i32, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp,
                                          i32, i64, i32, vp, vp, i32, f32, vp, vp, sz, vp, sz, vp]
        L.csa2_token_append.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, i64, vp]
        L.csa2_index_reindex_timed.argtypes = [vp, vp, vp, vp, SeqsC, i32, vp, i32, i32, i32, vp, vp, sz, vp, vp, vp,
                                               vp, vp]
        L.csa2_attend_timed.argtypes = [vp, vp, vp, SeqsC, vp, i32, vp, vp, i32, i64, i32, vp, i32, f32, vp, vp, sz,
                                        vp, vp, vp]
        L.csa2_window_append.argtypes = [vp, i64, vp, i64, vp, i32, i64, vp]
        L.csa2_stream_read_groups.argtypes = []
        L.csa2_stream_read_groups.restype = ctypes.c_int
        L.csa2_stream_read.argtypes = [vp, sz, vp, sz, vp, vp, vp]
        L.csa2_stream_read.restype = ctypes.c_int
        L.csa2_workspace_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
        L.csa2_workspace_bytes.restype = sz
        L.csa2_workspace_init.argtypes = [vp, sz, vp]
        L.csa2_status_string.argtypes = [ctypes.c_int]
        L.csa2_status_string.restype = ctypes.c_char_p
        L.csa2_version.argtypes = []
        for name in ("fp4_kv_append", "fp8_window_append", "csa2_index_full", "csa2_index_reindex", "csa2_attend",
                     "csa2_attend_fp8win", "csa2_workspace_init", "csa2_version", "mxfp4_key_append",
                     "csa2_index_full_mx", "csa2_index_full_mx_scan", "csa2_index_reindex_mx", "csa2_reindex_attend",
                     "csa2_index_full_scan_timed", "csa2_token_append", "csa2_window_append",
                     "csa2_index_reindex_timed", "csa2_attend_timed", "csa2_index_reindex_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise Csa2Error(fn, status, lib().csa2_status_string(status).decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensors passed to the CSA2 library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the CSA2 library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclass
class Seqs:
    """Where each query's context lives (mirrors csa2_seqs).

    kv_row0: int64 [n_q] device tensor; kv_len: int32 [n_q] device tensor;
    max_len_ub / total_len_ub: host bounds on the lengths; cache_rows: rows of the caches.
    """
    kv_row0: torch.Tensor
    kv_len: torch.Tensor
    max_len_ub: int
    total_len_ub: int
    cache_rows: int

    @property
    def n_q(self) -> int:
        return int(self.kv_len.numel())

    def c(self) -> SeqsC:
        if self.kv_row0.dtype != torch.int64 or self.kv_len.dtype != torch.int32:
            raise TypeError("kv_row0 must be int64 and kv_len int32")
        return SeqsC(_ptr(self.kv_row0), _ptr(self.kv_len), self.n_q, int(self.max_len_ub),
                     int(self.total_len_ub), int(self.cache_rows))


def fp4_kv_append(x, codes, scales, dst_rows=None, row0: int = 0, stream=None) -> None:
    """Quantise x (bf16 [n_tok, dim]) into rows of the FP4 cache (codes uint8 [rows, dim/2],
    scales uint8 [rows, dim/16])."""
    n_tok, dim = x.shape
    _check("fp4_kv_append", lib().fp4_kv_append(_ptr(x), n_tok, dim, _ptr(dst_rows), row0, _ptr(codes),
                                                _ptr(scales), codes.shape[0], _stream(stream)))


def fp8_window_append(x, out, dst_rows=None, row0: int = 0, stream=None) -> None:
    """Convert x (bf16 [n_tok, dim]) to E4M3 bytes in rows of an FP8 window store (uint8 [rows, dim])."""
    n_tok, dim = x.shape
    _check("fp8_window_append", lib().fp8_window_append(_ptr(x), n_tok, dim, _ptr(dst_rows), row0, _ptr(out),
                                                        out.shape[0], _stream(stream)))


def csa2_workspace_bytes(op: int, n_q: int, total_len_ub: int = 0, max_len_ub: int = 0, top_k: int = 0,
                         pool_blocks: int = 0) -> int:
    return int(lib().csa2_workspace_bytes(op, n_q, total_len_ub, max_len_ub, top_k, pool_blocks))


def csa2_workspace_init(ws, stream=None) -> None:
    _check("csa2_workspace_init", lib().csa2_workspace_init(_ptr(ws), ws.numel() * ws.element_size(),
                                                            _stream(stream)))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zeroed uint8 device workspace of at least nbytes (zeroed by the library's own kernel)."""
    if nbytes == SIZE_MAX:
        raise ValueError("workspace size query rejected the sizes")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    csa2_workspace_init(ws)
    return ws


def csa2_index_full(q_idx, w, k_idx, seqs: Seqs, top_k: int, pool_blocks: int, idx_out, pool_out, ws,
                    block: int = BLOCK, shared_kv: int = 0, stream=None) -> None:
    n_heads = q_idx.shape[1]
    _check("csa2_index_full", lib().csa2_index_full(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), seqs.c(), n_heads, top_k, block, pool_blocks, shared_kv,
        _ptr(idx_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream(stream)))


def csa2_index_full_prep(q_idx, w, k_idx, seqs: Seqs, top_k: int, pool_blocks: int, idx_out, pool_out, ws,
                         block: int = BLOCK, shared_kv: int = 0, stream=None) -> None:
    _check("csa2_index_full_prep", lib().csa2_index_full_prep(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), seqs.c(), q_idx.shape[1], top_k, block, pool_blocks, shared_kv,
        _ptr(idx_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream(stream)))


def csa2_index_full_scan(q_idx, w, k_idx, seqs: Seqs, top_k: int, pool_blocks: int, idx_out, pool_out, ws,
                         block: int = BLOCK, shared_kv: int = 0, stream=None) -> None:
    _check("csa2_index_full_scan", lib().csa2_index_full_scan(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), seqs.c(), q_idx.shape[1], top_k, block, pool_blocks, shared_kv,
        _ptr(idx_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream(stream)))


def csa2_index_full_select(q_idx, w, k_idx, seqs: Seqs, top_k: int, pool_blocks: int, idx_out, pool_out, ws,
                           block: int = BLOCK, shared_kv: int = 0, stream=None) -> None:
    _check("csa2_index_full_select", lib().csa2_index_full_select(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), seqs.c(), q_idx.shape[1], top_k, block, pool_blocks, shared_kv,
        _ptr(idx_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream(stream)))


def csa2_index_reindex(q_idx, w, k_idx, seqs: Seqs, pool, top_k: int, idx_out, ws, block: int = BLOCK,
                       stream=None) -> None:
    n_heads = q_idx.shape[1]
    _check("csa2_index_reindex", lib().csa2_index_reindex(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), seqs.c(), n_heads, _ptr(pool), pool.shape[1], block, top_k,
        _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))


def attend_workspace(n_q: int, top_k: int, window: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace for attention calls of these sizes (16 bytes when none is needed)."""
    return alloc_workspace(csa2_workspace_bytes(OP_ATTEND, n_q, 0, 0, top_k, window), device)


def _attend_ws(ws, q, top_k: int, window: int):
    # the caller's workspace, or (for one-off calls) a fresh zeroed one of the required size
    return ws if ws is not None else attend_workspace(q.shape[0], top_k, window, q.device)


def csa2_attend(q, codes, scales, seqs: Seqs, idx, swa, swa_row0, swa_cap: int, window: int,
                softmax_scale: float, out, win_new=None, ws=None, stream=None) -> None:
    """Attention over the selected FP4 entries and the bf16 window; win_new (bf16 [n_q, 128] or
    None): the new token's window vector, attended as position N - 1 and written to its row."""
    n_heads = q.shape[1]
    top_k = idx.shape[1] if idx is not None else 0
    swa_rows = swa.shape[0] if swa is not None else 0
    ws = _attend_ws(ws, q, top_k, window)
    _check("csa2_attend", lib().csa2_attend(
        _ptr(q), _ptr(codes), _ptr(scales), seqs.c(), _ptr(idx), top_k, _ptr(swa), _ptr(swa_row0), swa_cap,
        swa_rows, window, _ptr(win_new), n_heads, ctypes.c_float(softmax_scale), _ptr(out), _ptr(ws), ws.numel(),
        _stream(stream)))


def csa2_attend_fp8win(q, codes, scales, seqs: Seqs, idx, swa8, swa_row0, swa_cap: int, window: int,
                       softmax_scale: float, out, replay_start=None, win_new=None, ws=None, stream=None) -> None:
    n_heads = q.shape[1]
    top_k = idx.shape[1] if idx is not None else 0
    swa_rows = swa8.shape[0] if swa8 is not None else 0
    ws = _attend_ws(ws, q, top_k, window)
    _check("csa2_attend_fp8win", lib().csa2_attend_fp8win(
        _ptr(q), _ptr(codes), _ptr(scales), seqs.c(), _ptr(idx), top_k, _ptr(swa8), _ptr(swa_row0), swa_cap,
        swa_rows, window, _ptr(replay_start), _ptr(win_new), n_heads, ctypes.c_float(softmax_scale), _ptr(out),
        _ptr(ws), ws.numel(), _stream(stream)))


def csa2_reindex_attend(q_idx, w, k_idx, k_scales, seqs: Seqs, pool, top_k: int, idx_out, q, codes, scales, swa,
                        swa_row0, swa_cap: int, window: int, softmax_scale: float, out, ws, window_fp8: bool = False,
                        replay_start=None, win_new=None, att_ws=None, block: int = BLOCK, stream=None) -> None:
    """One Reindex layer in one call: selection inside the pool (bf16 keys, or MXFP4 keys when
    k_scales is given) and the attention over it.  att_ws: the attention workspace (None: a
    fresh one)."""
    swa_rows = swa.shape[0] if swa is not None else 0
    att_ws = _attend_ws(att_ws, q, top_k, window)
    _check("csa2_reindex_attend", lib().csa2_reindex_attend(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scales), seqs.c(), q_idx.shape[1], _ptr(pool), pool.shape[1], block,
        top_k, _ptr(idx_out), _ptr(q), _ptr(codes), _ptr(scales), _ptr(swa), 1 if window_fp8 else 0, _ptr(swa_row0),
        swa_cap, swa_rows, window, _ptr(replay_start), _ptr(win_new), q.shape[1], ctypes.c_float(softmax_scale),
        _ptr(out), _ptr(ws), ws.numel(), _ptr(att_ws), att_ws.numel(), _stream(stream)))


def csa2_token_append(x, dst_rows, codes, scales, k_new=None, k_idx=None, k_scales=None, stream=None) -> None:
    """The step's own token of a Full layer's set: x (bf16 [n_tok, 128]) into the FP4 cache and
    k_new (bf16 [n_tok, 64]) into the key cache (bf16 rows, or MXFP4 when k_scales is given)."""
    _check("csa2_token_append", lib().csa2_token_append(
        _ptr(x), _ptr(k_new), x.shape[0], _ptr(dst_rows), _ptr(codes), _ptr(scales), _ptr(k_idx), _ptr(k_scales),
        codes.shape[0], _stream(stream)))


def csa2_window_append(x, out, dst_rows=None, row0: int = 0, window_fp8: bool = False, stream=None) -> None:
    """Window vectors (bf16 [n_tok, 128]) into a window store (bf16 rows, or E4M3 bytes)."""
    _check("csa2_window_append", lib().csa2_window_append(
        _ptr(x), x.shape[0], _ptr(dst_rows), row0, _ptr(out), 1 if window_fp8 else 0, out.shape[0],
        _stream(stream)))


def mxfp4_key_append(x, codes, scales, dst_rows=None, row0: int = 0, stream=None) -> None:
    """Quantise x (bf16 [n_tok, dim]) into MXFP4 key rows (codes uint8 [rows, dim/2], scales uint8 [rows, dim/32])."""
    n_tok, dim = x.shape
    _check("mxfp4_key_append", lib().mxfp4_key_append(_ptr(x), n_tok, dim, _ptr(dst_rows), row0, _ptr(codes),
                                                      _ptr(scales), codes.shape[0], _stream(stream)))


def csa2_index_full_mx(q_idx, w, k_codes, k_scales, seqs: Seqs, top_k: int, pool_blocks: int, idx_out, pool_out,
                       ws, block: int = BLOCK, shared_kv: int = 0, stream=None) -> None:
    _check("csa2_index_full_mx", lib().csa2_index_full_mx(
        _ptr(q_idx), _ptr(w), _ptr(k_codes), _ptr(k_scales), seqs.c(), q_idx.shape[1], top_k, block, pool_blocks,
        shared_kv, _ptr(idx_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream(stream)))


def csa2_index_full_mx_scan(q_idx, w, k_codes, k_scales, seqs: Seqs, top_k: int, pool_blocks: int, idx_out,
                            pool_out, ws, block: int = BLOCK, shared_kv: int = 0, stream=None) -> None:
    _check("csa2_index_full_mx_scan", lib().csa2_index_full_mx_scan(
        _ptr(q_idx), _ptr(w), _ptr(k_codes), _ptr(k_scales), seqs.c(), q_idx.shape[1], top_k, block, pool_blocks,
        shared_kv, _ptr(idx_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream(stream)))


def csa2_index_full_scan_timed(q_idx, w, k_idx, k_scales, seqs: Seqs, top_k: int, pool_blocks: int, idx_out,
                               pool_out, ws, start_event, stop_event, block: int = BLOCK, shared_kv: int = 0,
                               stream=None) -> None:
    """The scan phase (k_scales None: bf16 keys; else MXFP4 codes in k_idx) with the scan kernel's
    start and end recorded into two torch.cuda.Event objects (recorded once already, so that
    their HIP events exist)."""
    _check("csa2_index_full_scan_timed", lib().csa2_index_full_scan_timed(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scales), seqs.c(), q_idx.shape[1], top_k, block, pool_blocks,
        shared_kv, _ptr(idx_out), _ptr(pool_out), _ptr(ws), ws.numel(), _stream(stream),
        ctypes.c_void_p(start_event.cuda_event), ctypes.c_void_p(stop_event.cuda_event)))


def _event(e):
    return ctypes.c_void_p(e.cuda_event) if e is not None else None


def csa2_index_reindex_noalloc(q_idx, w, k_idx, seqs: Seqs, pool, top_k: int, idx_out, block: int = BLOCK,
                               stream=None) -> None:
    """csa2_index_reindex with the library's static scratch in place of a workspace (n_q <= 64,
    pool_blocks <= 2048); allocates nothing."""
    _check("csa2_index_reindex_noalloc", lib().csa2_index_reindex_noalloc(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), seqs.c(), q_idx.shape[1], _ptr(pool), pool.shape[1], block, top_k,
        _ptr(idx_out), _stream(stream)))


def csa2_index_reindex_timed(q_idx, w, k_idx, k_scales, seqs: Seqs, pool, top_k: int, idx_out, ws, score_events,
                             select_events, block: int = BLOCK, stream=None) -> None:
    """csa2_index_reindex (or _mx with k_scales) with the scoring kernel's and the selection
    kernel's own start and end recorded into two pairs of torch.cuda.Event objects."""
    _check("csa2_index_reindex_timed", lib().csa2_index_reindex_timed(
        _ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(k_scales), seqs.c(), q_idx.shape[1], _ptr(pool), pool.shape[1], block,
        top_k, _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream), _event(score_events[0]), _event(score_events[1]),
        _event(select_events[0]), _event(select_events[1])))


def csa2_attend_timed(q, codes, scales, seqs: Seqs, idx, swa, swa_row0, swa_cap: int, window: int,
                      softmax_scale: float, out, start_event, stop_event, win_new=None, ws=None,
                      stream=None) -> None:
    """csa2_attend with the attention kernel's own start and end recorded into two torch events."""
    n_heads = q.shape[1]
    top_k = idx.shape[1] if idx is not None else 0
    swa_rows = swa.shape[0] if swa is not None else 0
    ws = _attend_ws(ws, q, top_k, window)
    _check("csa2_attend_timed", lib().csa2_attend_timed(
        _ptr(q), _ptr(codes), _ptr(scales), seqs.c(), _ptr(idx), top_k, _ptr(swa), _ptr(swa_row0), swa_cap,
        swa_rows, window, _ptr(win_new), n_heads, ctypes.c_float(softmax_scale), _ptr(out), _ptr(ws), ws.numel(),
        _stream(stream), _event(start_event), _event(stop_event)))


def csa2_stream_read(src, sink, start_event, stop_event, stream=None) -> None:
    """Measurement: a plain streaming read of src (device, 16-byte aligned) with the kernel's own
    start and end recorded into two torch events; sink: uint32 [csa2_stream_read_groups()]."""
    _check("csa2_stream_read", lib().csa2_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                                      sink.numel(), _stream(stream), _event(start_event),
                                                      _event(stop_event)))


def csa2_index_reindex_mx(q_idx, w, k_codes, k_scales, seqs: Seqs, pool, top_k: int, idx_out, ws,
                          block: int = BLOCK, stream=None) -> None:
    _check("csa2_index_reindex_mx", lib().csa2_index_reindex_mx(
        _ptr(q_idx), _ptr(w), _ptr(k_codes), _ptr(k_scales), seqs.c(), q_idx.shape[1], _ptr(pool), pool.shape[1],
        block, top_k, _ptr(idx_out), _ptr(ws), ws.numel(), _stream(stream)))
