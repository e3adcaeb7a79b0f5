"""The CSA2 workloads this library is built and measured on, and a driver that runs one decode
step (or one prefill chunk) of a workload through the C ABI.  Workloads 0-4 are the five
configurations of the problem statement; 5-7 are the 1M-context decode with the pages' storage
formats of section XI of [Article]: an FP8 window store with SWA Bounded Replay starts (5),
MXFP4 indexer keys (6), and both (7); 8 is a prefill chunk through a Full layer that gives every
query token its own block pool, two Reindex layers inside those pools and a Reuse layer.

Mode schedule ([Article] "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per
Token", section VIII, and the [Summary] page's Technical Approach):
  F  Full     - own indexer query over its own (owned) keys; Top-K over the whole context;
                the first Full layer of a pool-using schedule also builds the block pool;
  R  Reindex  - own indexer query over the most recent Full layer's keys, Top-K inside the pool;
  U  Reuse    - inherits the most recent index-producing layer's Top-K (no indexer launch).
Every layer has its own attention query and its own sliding-window store.  Layer sequencing is
host code; all computation runs in the library's kernels.

Inputs are synthetic (compressed_sparse_attention_07_amd.synth); the library and this driver
never read anything else.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import csa2 as C
from . import synth


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    context: int | None            # per-sequence context N (decode); None for ragged
    layers: str                    # mode letters, one per layer
    pool_blocks: int
    top_k: int = 512
    window: int = 128
    heads: int = 16
    idx_heads: int = 4
    prefill_chunk: int = 0         # > 0: a prefill chunk of this many new tokens on a `context` cache
    ragged: tuple | None = None    # (lo, hi) for log-uniform per-sequence lengths
    appends: bool = True           # decode appends the new token's KV (one vector per owned set)
    window_fp8: bool = False       # window stores hold E4M3 bytes ([Article] XI) and attention takes
                                   # per-sequence replay starts ([Article] XII): even sequences replay
                                   # their last replay_tail positions, odd ones have no bound
    replay_tail: int = 64
    keys_mx: bool = False          # indexer keys stored as MXFP4 ([Article] XI: E2M1 + E8M0 per 32
                                   # channels); the step also appends each new token's key

    def lengths(self) -> np.ndarray:
        if self.ragged:
            return synth.log_uniform_lengths(self.wid, self.batch, self.ragged[0], self.ragged[1])
        return np.full(self.batch, self.context, dtype=np.int64)


def c2_layers(n=20):
    s = "F"
    while len(s) < n:
        s += "RRUUU"
    return s[:n]


WORKLOADS = {
    0: Workload(0, "decode_b1_4k_1layer", 1, 4096, "F", 256),
    1: Workload(1, "decode_b32_64k_8layers", 32, 65536, "FRRRUUUU", 2048),
    2: Workload(2, "decode_b8_1m_20layers", 8, 1 << 20, c2_layers(20), 2048),
    3: Workload(3, "prefill_4096_on_128k", 1, 131072, "F", 0, prefill_chunk=4096, appends=True),
    4: Workload(4, "decode_b64_ragged_1k_1m_4layers", 64, None, "FUFU", 0, ragged=(1024, 1 << 20)),
    5: Workload(5, "decode_b8_1m_20layers_fp8win_replay", 8, 1 << 20, c2_layers(20), 2048, window_fp8=True),
    6: Workload(6, "decode_b8_1m_20layers_mxkeys", 8, 1 << 20, c2_layers(20), 2048, keys_mx=True),
    7: Workload(7, "decode_b8_1m_20layers_mxkeys_fp8win_replay", 8, 1 << 20, c2_layers(20), 2048,
                window_fp8=True, keys_mx=True),
    8: Workload(8, "prefill_4096_on_128k_4layers", 1, 131072, "FRRU", 2048, prefill_chunk=4096, appends=True),
}


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


@dataclass
class KvSet:
    """One owned main-KV set (FP4) plus its indexer keys, sequences back to back.  The keys are
    bf16 rows (k_idx) or MXFP4 rows (k_codes [rows, 32] + k_scales [rows, 2]), never both."""
    codes: torch.Tensor
    scales: torch.Tensor
    k_idx: torch.Tensor | None
    x_new: torch.Tensor       # bf16 [B, 128]: the step's new token per sequence (post-RoPE)
    new_rows: torch.Tensor    # int64 [B]: row each new token is written to
    k_codes: torch.Tensor | None = None
    k_scales: torch.Tensor | None = None
    k_new: torch.Tensor | None = None    # bf16 [B, 64]: the step's new indexer key

    def clone(self) -> "KvSet":
        c = lambda t: None if t is None else t.clone()
        return KvSet(self.codes.clone(), self.scales.clone(), c(self.k_idx), self.x_new, self.new_rows,
                     c(self.k_codes), c(self.k_scales), self.k_new)


@dataclass
class Layer:
    mode: str
    kv_set: int
    q: torch.Tensor                  # bf16 [n_q, H, 128]
    swa: torch.Tensor                # bf16 [n_q * swa_cap, 128], or E4M3 bytes when the window is FP8
    win_new: torch.Tensor | None = None   # decode: bf16 [n_q, 128], the step's own window vector per query
    win_chunk: torch.Tensor | None = None  # prefill: bf16 [T, 128], the chunk's window vectors
    win_rows: torch.Tensor | None = None   # prefill: int64 [T], their store rows
    q_idx: torch.Tensor | None = None
    w: torch.Tensor | None = None
    idx: torch.Tensor | None = None  # output of F/R layers
    idx_src: int = -1                # layer whose idx a U layer attends with
    out: torch.Tensor | None = None


class Runner:
    """Device state of one workload and its step.  host copies of the inputs are kept in
    `self.host` when keep_host=True (for the oracle checks in tests and the bench baseline)."""

    def __init__(self, wl: Workload, device="cuda", keep_host=False, seed=0, copies=1, fused_reindex=False):
        """copies > 1 keeps that many device copies of the KV sets (identical values); step() then
        rotates through them so consecutive steps never re-read a set that a last-level cache
        could still hold.  fused_reindex: Reindex layers run as one csa2_reindex_attend call (the
        same three kernels as csa2_index_reindex + csa2_attend, issued by one entry point)."""
        self.wl = wl
        self.fused_reindex = fused_reindex
        self.device = device
        self.host = {} if keep_host else None
        B = wl.batch
        lengths = wl.lengths()
        if wl.prefill_chunk:
            T = wl.prefill_chunk
            total_rows = wl.context + T
            self.n_q = T
            self.seq_len = np.array([total_rows], dtype=np.int64)
            self.seq_row0 = np.zeros(1, dtype=np.int64)
            q_len = wl.context + 1 + np.arange(T, dtype=np.int64)      # token t sees [0, C + t]
            q_row0 = np.zeros(T, dtype=np.int64)
        else:
            self.n_q = B
            self.seq_len = lengths
            self.seq_row0 = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
            total_rows = int(lengths.sum())
            q_len = lengths
            q_row0 = self.seq_row0
        self.q_len = q_len
        self.q_row0 = q_row0
        self.rows = total_rows
        self.seqs = C.Seqs(kv_row0=torch.from_numpy(q_row0).to(device),
                           kv_len=torch.from_numpy(q_len.astype(np.int32)).to(device),
                           max_len_ub=int(q_len.max()), total_len_ub=int(q_len.sum()), cache_rows=total_rows)
        wid = wl.wid
        # owned KV sets: one per Full layer
        full_layers = [i for i, m in enumerate(wl.layers) if m == "F"]
        self.sets = []
        for s_i, _ in enumerate(full_layers):
            sig = synth.channel_sigma(wid, synth.T_KV_SIGMA, 128, seq=s_i)
            x = synth.kv_bf16(wid, synth.T_KV, total_rows, 128, sig, seq=s_i)
            k = synth.int_bf16(wid, synth.T_IDX_K, (total_rows, 64), seq=s_i)
            codes = torch.empty((total_rows, 64), dtype=torch.uint8, device=device)
            scales = torch.empty((total_rows, 8), dtype=torch.uint8, device=device)
            if wl.prefill_chunk:
                new_rows = np.arange(wl.context, total_rows, dtype=np.int64)
            else:
                new_rows = self.seq_row0 + lengths - 1                 # the step's own token
            # the cache before the step: every row but the new tokens' rows
            x_dev = bf16_dev(x, device)
            C.fp4_kv_append(x_dev, codes, scales)
            new_rows_t = torch.from_numpy(new_rows).to(device)
            x_new = x_dev[new_rows_t].contiguous()
            del x_dev
            k_dev = bf16_dev(k, device)
            k_new = k_dev[new_rows_t].contiguous()
            if wl.keys_mx:   # keys written by the library's MXFP4 append; the bf16 rows are dropped
                kc = torch.empty((total_rows, 32), dtype=torch.uint8, device=device)
                ks = torch.empty((total_rows, 2), dtype=torch.uint8, device=device)
                C.mxfp4_key_append(k_dev, kc, ks)
                st = KvSet(codes, scales, None, x_new, new_rows_t, kc, ks, k_new)
            else:
                st = KvSet(codes, scales, k_dev, x_new, new_rows_t, k_new=k_new)
            del k_dev
            self.sets.append(st)
            if self.host is not None:
                self.host.setdefault("x", []).append(x)
                self.host.setdefault("k_idx", []).append(k)
                self.host.setdefault("new_rows", []).append(new_rows)
            del x, k
        # Scramble the new tokens' rows so the step's append is what makes them correct.
        # (A key row becomes +6 * 2^10 (MXFP4) or 100 (bf16) in every channel: a large score, so a
        # missing key write would change the selection.)
        for st in self.sets:
            st.codes[st.new_rows] = 0xEE
            st.scales[st.new_rows] = 0x77
            if st.k_codes is not None:
                st.k_codes[st.new_rows] = 0x77
                st.k_scales[st.new_rows] = 127 + 10
            if st.k_idx is not None:
                st.k_idx[st.new_rows] = 100.0
        self.copies = [self.sets]
        for _ in range(1, copies):
            self.copies.append([st.clone() for st in self.sets])
        self._next_copy = 0
        # layers
        self.swa_cap = wl.window + (wl.prefill_chunk or 0)
        self.layers = []
        cur_set, last_idx = -1, -1
        for l, m in enumerate(wl.layers):
            if m == "F":
                cur_set += 1
            q = synth.normal_bf16(wid, synth.T_Q, (self.n_q, wl.heads, 128), seq=l)
            ssig = synth.channel_sigma(wid, synth.T_SWA_SIGMA, 128, seq=l)
            swa = synth.kv_bf16(wid, synth.T_SWA, self.n_q_swa() * self.swa_cap, 128, ssig, seq=l)
            # The rows the step writes (decode: each query's position N - 1; prefill: the chunk's
            # own positions) hold the step's vectors in the host copy (the store after the step)
            # and a marker on the device until the step writes them (bf16 1000 / E4M3 448: a
            # missing write would dominate the attention).
            if wl.prefill_chunk:
                new_pos = wl.context + np.arange(wl.prefill_chunk, dtype=np.int64)
                new_row = new_pos % self.swa_cap
                win_vec = swa[new_row]
            else:
                new_row = np.arange(self.n_q, dtype=np.int64) * self.swa_cap + (q_len - 1) % self.swa_cap
                win_vec = synth.kv_bf16(wid, synth.T_SWA_NEW, self.n_q, 128, ssig, seq=l)
                swa[new_row] = win_vec
            self.win_rows_host = new_row                                  # the same rows in every layer
            swa_before = swa.copy()
            swa_before[new_row] = 0x447A                                  # bf16 1000.0
            swa_dev = bf16_dev(swa_before, device)
            if wl.window_fp8:  # the window store is written by the library's FP8 append
                swa8 = torch.empty(swa_dev.shape, dtype=torch.uint8, device=device)
                C.fp8_window_append(swa_dev, swa8)
                swa_dev = swa8
            L = Layer(m, cur_set, bf16_dev(q, device), swa_dev)
            if wl.prefill_chunk:
                L.win_chunk = bf16_dev(win_vec, device)
                L.win_rows = torch.from_numpy(new_row).to(device)
            else:
                L.win_new = bf16_dev(win_vec, device)
            if m in "FR":
                qi = synth.int_bf16(wid, synth.T_IDX_Q, (self.n_q, wl.idx_heads, 64), seq=l)
                w = synth.int_weights(wid, synth.T_IDX_W, (self.n_q, wl.idx_heads), seq=l)
                L.q_idx = bf16_dev(qi, device)
                L.w = torch.from_numpy(w).to(device)
                L.idx = torch.empty((self.n_q, wl.top_k), dtype=torch.int32, device=device)
                last_idx = l
                if self.host is not None:
                    self.host.setdefault("q_idx", {})[l] = qi
                    self.host.setdefault("w", {})[l] = w
            else:
                L.idx_src = last_idx
            L.out = torch.empty((self.n_q, wl.heads, 128), dtype=torch.float32, device=device)
            if self.host is not None:
                self.host.setdefault("q", {})[l] = q
                self.host.setdefault("swa", {})[l] = swa
            self.layers.append(L)
        # per-query window ring: decode = one ring of `window` rows per sequence;
        # prefill = one shared store holding positions C-W .. C+T-1 (position p at row p mod cap)
        if wl.prefill_chunk:
            self.swa_row0 = torch.zeros(self.n_q, dtype=torch.int64, device=device)
        else:
            self.swa_row0 = torch.arange(self.n_q, dtype=torch.int64, device=device) * self.swa_cap
        self.pool = torch.empty((self.n_q, max(wl.pool_blocks, 1)), dtype=torch.int32, device=device) \
            if wl.pool_blocks else None
        # replay starts of the FP8-window workload: even sequences replayed their last replay_tail positions
        self.replay = None
        if wl.window_fp8:
            rs = np.where(np.arange(self.n_q) % 2 == 0, np.maximum(q_len - wl.replay_tail, 0), 0).astype(np.int64)
            self.replay_host = rs
            self.replay = torch.from_numpy(rs).to(device)
        # workspaces: one per op kind (each op's prefix is sized by n_q)
        self.ws_full = C.alloc_workspace(C.csa2_workspace_bytes(
            C.OP_INDEX_FULL, self.n_q, self.seqs.total_len_ub, self.seqs.max_len_ub, wl.top_k, wl.pool_blocks))
        self.ws_re = C.alloc_workspace(C.csa2_workspace_bytes(
            C.OP_INDEX_REINDEX, self.n_q, 0, 0, wl.top_k, max(wl.pool_blocks, 1))) if "R" in wl.layers else None
        self.ws_att = C.attend_workspace(self.n_q, wl.top_k, wl.window)
        self.scale = 1.0 / math.sqrt(128.0)
        torch.cuda.synchronize()

    def n_q_swa(self) -> int:
        return 1 if self.wl.prefill_chunk else self.n_q

    def step(self, stream=None, timing=None, copy=None) -> None:
        """One pass of the hot path: append the step's KV, then every layer in order.
        timing: optional dict; the Full-mode scan ("scan"), the two kernels of each separate Reindex
        selection ("reindex_score", "reindex_select") and each bf16-window attention ("attend") then
        record their own start and end into a torch.cuda.Event pair appended to timing[kind] (for
        timing those kernels inside a timed loop; not for graph capture).
        copy: which device copy of the KV sets to use (default: the next one in rotation)."""
        wl = self.wl
        if copy is None:
            copy = self._next_copy
            self._next_copy = (self._next_copy + 1) % len(self.copies)
        self.sets = self.copies[copy]
        if wl.appends:   # the step's own token: FP4 KV row and indexer key row of every owned set
            for st in self.sets:
                C.csa2_token_append(st.x_new, st.new_rows, st.codes, st.scales, k_new=st.k_new,
                                    k_idx=st.k_codes if wl.keys_mx else st.k_idx,
                                    k_scales=st.k_scales if wl.keys_mx else None, stream=stream)
        def ev_pair(kind):
            # the two records only create the events; the kernels' launches record into them
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            e1.record()
            timing.setdefault(kind, []).append((e0, e1))
            return e0, e1

        pool_built = False
        for L in self.layers:
            st = self.sets[L.kv_set]
            if L.win_chunk is not None:   # a prefill chunk's own window entries, before they are read
                C.csa2_window_append(L.win_chunk, L.swa, dst_rows=L.win_rows, window_fp8=wl.window_fp8, stream=stream)
            if L.mode == "F":
                want_pool = wl.pool_blocks if (self.pool is not None and not pool_built) else 0
                pool = self.pool if want_pool else None
                shared = 1 if wl.prefill_chunk else 0   # a prefill chunk: all queries read one sequence
                keys = st.k_codes if wl.keys_mx else st.k_idx    # prep and select read no keys
                C.csa2_index_full_prep(L.q_idx, L.w, keys, self.seqs, wl.top_k, want_pool, L.idx, pool,
                                       self.ws_full, shared_kv=shared, stream=stream)
                if timing is not None:
                    e0, e1 = ev_pair("scan")
                    C.csa2_index_full_scan_timed(L.q_idx, L.w, st.k_codes if wl.keys_mx else st.k_idx,
                                                 st.k_scales if wl.keys_mx else None, self.seqs, wl.top_k, want_pool,
                                                 L.idx, pool, self.ws_full, e0, e1, shared_kv=shared, stream=stream)
                elif wl.keys_mx:
                    C.csa2_index_full_mx_scan(L.q_idx, L.w, st.k_codes, st.k_scales, self.seqs, wl.top_k, want_pool,
                                              L.idx, pool, self.ws_full, shared_kv=shared, stream=stream)
                else:
                    C.csa2_index_full_scan(L.q_idx, L.w, st.k_idx, self.seqs, wl.top_k, want_pool, L.idx, pool,
                                           self.ws_full, shared_kv=shared, stream=stream)
                C.csa2_index_full_select(L.q_idx, L.w, keys, self.seqs, wl.top_k, want_pool, L.idx, pool,
                                         self.ws_full, shared_kv=shared, stream=stream)
                pool_built = pool_built or want_pool > 0
                idx = L.idx
            elif L.mode == "R" and self.fused_reindex and timing is None:
                C.csa2_reindex_attend(L.q_idx, L.w, st.k_codes if wl.keys_mx else st.k_idx,
                                      st.k_scales if wl.keys_mx else None, self.seqs, self.pool, wl.top_k, L.idx, L.q,
                                      st.codes, st.scales, L.swa, self.swa_row0, self.swa_cap, wl.window, self.scale,
                                      L.out, self.ws_re, window_fp8=wl.window_fp8, replay_start=self.replay,
                                      win_new=L.win_new, att_ws=self.ws_att, stream=stream)
                continue
            elif L.mode == "R" and timing is not None:
                C.csa2_index_reindex_timed(L.q_idx, L.w, st.k_codes if wl.keys_mx else st.k_idx,
                                           st.k_scales if wl.keys_mx else None, self.seqs, self.pool, wl.top_k, L.idx,
                                           self.ws_re, ev_pair("reindex_score"), ev_pair("reindex_select"),
                                           stream=stream)
                idx = L.idx
            elif L.mode == "R":
                if wl.keys_mx:
                    C.csa2_index_reindex_mx(L.q_idx, L.w, st.k_codes, st.k_scales, self.seqs, self.pool, wl.top_k,
                                            L.idx, self.ws_re, stream=stream)
                else:
                    C.csa2_index_reindex(L.q_idx, L.w, st.k_idx, self.seqs, self.pool, wl.top_k, L.idx, self.ws_re,
                                         stream=stream)
                idx = L.idx
            else:
                idx = self.layers[L.idx_src].idx
            if wl.window_fp8:
                C.csa2_attend_fp8win(L.q, st.codes, st.scales, self.seqs, idx, L.swa, self.swa_row0, self.swa_cap,
                                     wl.window, self.scale, L.out, replay_start=self.replay, win_new=L.win_new,
                                     ws=self.ws_att, stream=stream)
            elif timing is not None:
                e0, e1 = ev_pair("attend")
                C.csa2_attend_timed(L.q, st.codes, st.scales, self.seqs, idx, L.swa, self.swa_row0, self.swa_cap,
                                    wl.window, self.scale, L.out, e0, e1, win_new=L.win_new, ws=self.ws_att,
                                    stream=stream)
            else:
                C.csa2_attend(L.q, st.codes, st.scales, self.seqs, idx, L.swa, self.swa_row0, self.swa_cap,
                              wl.window, self.scale, L.out, win_new=L.win_new, ws=self.ws_att, stream=stream)

    def capture(self):
        """Capture one step per KV copy into HIP graphs (torch.cuda.CUDAGraph on torch's current
        device).  Returns the list of graphs; replaying graph k runs the step on copy k.  The
        kernels issue no memset, and workspaces were zeroed when allocated, outside capture."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for k in range(len(self.copies)):
                self.step(copy=k)
        torch.cuda.current_stream().wait_stream(side)
        graphs = []
        for k in range(len(self.copies)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(copy=k)
            graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    # ---- accounting of the bytes the method itself must move per step ----
    def kernel_bytes(self) -> dict:
        """Algorithmic bytes of ONE launch of each timed kernel: "scan" (every visible key once),
        "reindex_score" (every pool position's key read, its 4-B order key written),
        "reindex_select" (those order keys read back), "attend" (72 B per selected FP4 entry + one window entry per
        window position + the query, the new window vector read and written, the output), and
        "kv_gather" (the attention's cache gathers alone: selected entries and window entries)."""
        wl = self.wl
        key_bytes = 34 if wl.keys_mx else 128
        win_entry = 128 if wl.window_fp8 else 256
        win = np.minimum(self.q_len, wl.window)
        if wl.window_fp8:
            win = np.minimum(win, self.q_len - self.replay_host)
        sel = np.minimum(self.q_len, wl.top_k)
        gather = int(sel.sum()) * 72 + int(win.sum()) * win_entry
        new_vec = 0 if wl.prefill_chunk else self.n_q * (256 + win_entry)
        cand = self.n_q * min(wl.pool_blocks * 8, int(self.q_len.max())) if wl.pool_blocks else 0
        return {"scan": int(self.q_len.sum()) * key_bytes,
                "reindex_score": cand * (key_bytes + 4),
                "reindex_select": cand * 4,
                "attend": gather + self.n_q * wl.heads * 128 * (2 + 4) + new_vec,
                "kv_gather": gather}

    def algorithmic_bytes(self) -> dict:
        """Bytes per step by kernel family (see the design notes for the per-unit figures)."""
        wl = self.wl
        n_sum = int(self.q_len.sum())
        out = {"append": 0, "index_full": 0, "index_reindex": 0, "attend": 0}
        n_sets = len(self.sets)
        key_bytes = 34 if wl.keys_mx else 128                     # MXFP4 or bf16 indexer key
        win_entry = 128 if wl.window_fp8 else 256                    # E4M3 or bf16 window entry
        if wl.appends:   # per token and owned set: KV in + FP4 out, key in + key out
            toks = (wl.prefill_chunk or self.n_q) * n_sets
            out["append"] = toks * (256 + 72 + 128 + (34 if wl.keys_mx else 128))
        # every layer writes its own window entries: the step's token (decode) or the chunk's tokens
        out["append"] += len(self.layers) * (wl.prefill_chunk or self.n_q) * (256 + win_entry)
        for L in self.layers:
            if L.mode == "F":
                out["index_full"] += n_sum * key_bytes             # every visible indexer key, once
            elif L.mode == "R":
                cand = self.n_q * min(wl.pool_blocks * 8, int(self.q_len.max()))
                out["index_reindex"] += cand * key_bytes
            win = np.minimum(self.q_len, wl.window)
            win_bytes = 256                                         # bf16 window entry
            if wl.window_fp8:
                win = np.minimum(win, self.q_len - self.replay_host)
                win_bytes = 128                                     # E4M3 window entry
            sel = np.minimum(self.q_len, wl.top_k)
            out["attend"] += int(sel.sum()) * 72 + int(win.sum()) * win_bytes + self.n_q * wl.heads * 128 * (2 + 4)
        return out
