"""CPU checks of the C ABI library: it loads, exports every function include/*.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed: every call here
fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

from compressed_sparse_attention_07_amd import csa2 as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def declared_functions():
    names = set()
    for hp in HEADERS:
        text = open(hp).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fp4_kv_append", "csa2_index_full", "csa2_index_reindex", "csa2_attend"):
        assert n in names
    assert set(names) == set(C.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    L = C.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert L.csa2_version() == 100
    for s in range(8):
        assert L.csa2_status_string(s)


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: each call below fails validation first


def seqs(n_q=2, max_len=100, total=200, rows=200, row0=FAKE, kl=FAKE):
    return C.SeqsC(row0, kl, n_q, max_len, total, rows)


def test_append_validation():
    L = C.lib()
    assert L.fp4_kv_append(FAKE, 10, 100, None, 0, FAKE, FAKE, 10, None) == C.ERR_SHAPE      # dim % 16
    assert L.fp4_kv_append(FAKE, -1, 128, None, 0, FAKE, FAKE, 10, None) == C.ERR_SHAPE
    assert L.fp4_kv_append(FAKE, 0, 128, None, 0, FAKE, FAKE, 10, None) == C.OK              # no-op
    assert L.fp4_kv_append(None, 5, 128, None, 0, FAKE, FAKE, 10, None) == C.ERR_NULL
    assert L.fp4_kv_append(FAKE, 5, 128, None, 6, FAKE, FAKE, 10, None) == C.ERR_CAPACITY
    assert L.fp4_kv_append(ctypes.c_void_p(0x10008), 5, 128, None, 0, FAKE, FAKE, 10, None) == C.ERR_SHAPE


def test_index_full_validation():
    L = C.lib()
    ws_need = C.csa2_workspace_bytes(C.OP_INDEX_FULL, 2, 200, 100, 512, 256)
    assert ws_need > 0
    args = dict(q=FAKE, w=FAKE, k=FAKE)

    def call(s=None, heads=4, top_k=512, block=8, pool=256, idx=FAKE, pool_out=FAKE, ws=FAKE, ws_bytes=ws_need):
        return L.csa2_index_full(args["q"], args["w"], args["k"], s or seqs(), heads, top_k, block, pool, 0, idx,
                                 pool_out, ws, ws_bytes, None)

    assert call(heads=0) == C.ERR_SHAPE
    assert call(heads=9) == C.ERR_SHAPE
    assert call(top_k=0) == C.ERR_SHAPE
    assert call(top_k=4097) == C.ERR_SHAPE
    assert call(pool=-1) == C.ERR_SHAPE
    assert call(block=16) == C.ERR_UNSUPPORTED
    assert call(idx=None) == C.ERR_NULL
    assert call(pool_out=None) == C.ERR_NULL
    assert call(ws=None) == C.ERR_WORKSPACE
    assert call(ws_bytes=ws_need - 1) == C.ERR_WORKSPACE
    assert call(s=seqs(row0=None)) == C.ERR_NULL
    assert call(s=seqs(n_q=-1)) == C.ERR_SHAPE
    assert call(s=seqs(n_q=0)) == C.OK


def test_reindex_and_attend_validation():
    L = C.lib()
    need_r = C.csa2_workspace_bytes(C.OP_INDEX_REINDEX, 2, 0, 0, 512, 2048)
    assert need_r > 0
    assert L.csa2_index_reindex(FAKE, FAKE, FAKE, seqs(), 4, FAKE, 0, 8, 512, FAKE, FAKE, need_r, None) == C.ERR_SHAPE
    assert L.csa2_index_reindex(FAKE, FAKE, FAKE, seqs(), 4, None, 2048, 8, 512, FAKE, FAKE, need_r, None) == C.ERR_NULL
    assert L.csa2_index_reindex(FAKE, FAKE, FAKE, seqs(), 4, FAKE, 2048, 8, 512, FAKE, FAKE, need_r - 1,
                                None) == C.ERR_WORKSPACE
    need_a = C.csa2_workspace_bytes(C.OP_ATTEND, 2, 0, 0, 512, 128)
    assert need_a >= 2 * 5 * (16 * 130 * 4)     # five partials of 16 heads x (128 + max + sum) per query

    def att(top_k=512, window=128, cap=128, heads=16, scale=0.1, idx=FAKE, swa=FAKE, swa_rows=1000, win_new=None,
            ws=FAKE, ws_bytes=None):
        return L.csa2_attend(FAKE, FAKE, FAKE, seqs(), idx, top_k, swa, FAKE, cap, swa_rows, window, win_new, heads,
                             ctypes.c_float(scale), FAKE, ws, need_a if ws_bytes is None else ws_bytes, None)

    assert att(ws=None) == C.ERR_WORKSPACE
    assert att(ws_bytes=need_a - 1) == C.ERR_WORKSPACE
    assert att(ws=ctypes.c_void_p(0x10008)) == C.ERR_WORKSPACE   # 16-byte aligned

    assert att(heads=17) == C.ERR_SHAPE
    assert att(cap=100) == C.ERR_SHAPE          # the window ring must hold the window
    assert att(top_k=0, window=0) == C.ERR_SHAPE
    assert att(scale=float("nan")) == C.ERR_SHAPE
    assert att(idx=None) == C.ERR_NULL
    assert att(swa=None) == C.ERR_NULL
    assert att(swa_rows=1 << 31) == C.ERR_SHAPE
    assert att(top_k=4097) == C.ERR_SHAPE
    assert att(window=4097, cap=5000) == C.ERR_SHAPE
    assert att(win_new=ctypes.c_void_p(0x10008)) == C.ERR_SHAPE   # the new window vector must be 16-byte aligned


def test_reindex_attend_validation():
    # every check of both halves runs before anything is launched
    L = C.lib()
    need_r = C.csa2_workspace_bytes(C.OP_INDEX_REINDEX, 2, 0, 0, 512, 2048)

    need_a = C.csa2_workspace_bytes(C.OP_ATTEND, 2, 0, 0, 512, 128)

    def call(pool_blocks=2048, top_k=512, idx_heads=4, heads=16, window=128, cap=128, fp8=0, k_scales=None,
             idx_out=FAKE, q=FAKE, swa=FAKE, ws_bytes=need_r, s=None, att_ws=FAKE, att_bytes=need_a):
        return L.csa2_reindex_attend(FAKE, FAKE, FAKE, k_scales, s or seqs(), idx_heads, FAKE, pool_blocks, 8, top_k,
                                     idx_out, q, FAKE, FAKE, swa, fp8, FAKE, cap, 1000, window, None, None, heads,
                                     ctypes.c_float(0.1), FAKE, FAKE, ws_bytes, att_ws, att_bytes, None)

    assert call(pool_blocks=0) == C.ERR_SHAPE
    assert call(idx_heads=9) == C.ERR_SHAPE
    assert call(heads=17) == C.ERR_SHAPE
    assert call(cap=100) == C.ERR_SHAPE
    assert call(fp8=2) == C.ERR_SHAPE
    assert call(idx_out=None) == C.ERR_NULL
    assert call(q=None) == C.ERR_NULL
    assert call(swa=None) == C.ERR_NULL
    assert call(ws_bytes=need_r - 1) == C.ERR_WORKSPACE
    assert call(att_ws=None) == C.ERR_WORKSPACE                    # the attention workspace is checked too
    assert call(att_bytes=need_a - 1) == C.ERR_WORKSPACE
    assert call(k_scales=ctypes.c_void_p(0x10001)) == C.ERR_SHAPE    # MXFP4 scales must be 2-byte aligned
    assert call(s=seqs(n_q=0)) == C.OK


def test_token_and_window_append_validation():
    L = C.lib()
    def tok(n=4, x=FAKE, k_new=None, dst=FAKE, codes=FAKE, scales=FAKE, k_idx=None, cap=100):
        return L.csa2_token_append(x, k_new, n, dst, codes, scales, k_idx, None, cap, None)
    assert tok(n=-1) == C.ERR_SHAPE
    assert tok(n=0, x=None) == C.OK                          # nothing to do
    assert tok(x=None) == C.ERR_NULL
    assert tok(dst=None) == C.ERR_NULL                       # the decode step names its rows
    assert tok(k_new=FAKE, k_idx=None) == C.ERR_NULL         # a key needs its cache
    assert tok(x=ctypes.c_void_p(0x10008)) == C.ERR_SHAPE    # 16-byte aligned input
    assert tok(codes=ctypes.c_void_p(0x10004)) == C.ERR_SHAPE

    def win(n=4, x=FAKE, dst=None, row0=0, out=FAKE, fp8=0, cap=100):
        return L.csa2_window_append(x, n, dst, row0, out, fp8, cap, None)
    assert win(fp8=2) == C.ERR_SHAPE
    assert win(out=None) == C.ERR_NULL
    assert win(row0=98) == C.ERR_CAPACITY                    # rows 98..101 past a 100-row store
    assert win(out=ctypes.c_void_p(0x10008)) == C.ERR_SHAPE
    assert win(n=0, x=None) == C.OK


def test_stream_read_validation():
    L = C.lib()
    sink = ctypes.c_void_p(0x20000)
    assert L.csa2_stream_read(None, 1 << 20, sink, 4096, None, None, None) == C.ERR_NULL
    assert L.csa2_stream_read(FAKE, 1 << 20, None, 4096, None, None, None) == C.ERR_NULL
    assert L.csa2_stream_read(ctypes.c_void_p(0x10008), 1 << 20, sink, 4096, None, None, None) == C.ERR_SHAPE
    assert L.csa2_stream_read(FAKE, (1 << 20) + 4, sink, 4096, None, None, None) == C.ERR_SHAPE
    assert L.csa2_stream_read(FAKE, 0, sink, 4096, None, None, None) == C.ERR_SHAPE


def test_workspace_sizes():
    # Full: grows with the context bound; Reindex: with pool size only; Attend: with splits
    a = C.csa2_workspace_bytes(C.OP_INDEX_FULL, 8, 8 << 20, 1 << 20, 512, 2048)
    b = C.csa2_workspace_bytes(C.OP_INDEX_FULL, 8, 16 << 20, 2 << 20, 512, 2048)
    assert 0 < a < b
    assert a >= 8 * (1 << 20) * 8          # 4 B key + 4 B candidate per position
    assert C.csa2_workspace_bytes(C.OP_INDEX_FULL, 8, 100, 10, 0, 0) == C.SIZE_MAX
    r = C.csa2_workspace_bytes(C.OP_INDEX_REINDEX, 8, 0, 0, 512, 2048)
    assert r >= 8 * 2048 * 8 * 4          # a 4 B key per pool position
    a8 = C.csa2_workspace_bytes(C.OP_ATTEND, 8, 0, 0, 512, 128)
    assert a8 >= 8 * 5 * (16 * 130 * 4) and a8 < C.csa2_workspace_bytes(C.OP_ATTEND, 8, 0, 0, 1024, 128)
    assert C.csa2_workspace_bytes(C.OP_ATTEND, 65, 0, 0, 512, 128) == 0    # more than 64 queries: no split
    assert C.csa2_workspace_bytes(C.OP_ATTEND, 8, 0, 0, 64, 0) == 0        # one workgroup covers a query
    assert C.csa2_workspace_bytes(C.OP_ATTEND, 8, 0, 0, 512, 5000) == C.SIZE_MAX
    assert C.csa2_workspace_bytes(99, 8, 0, 0, 1, 1) == C.SIZE_MAX
