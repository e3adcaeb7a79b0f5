"""Shared setup for the GPU parity tests: seeded inputs go to both the HIP path (through the
C ABI binding) and the CPU oracle; nothing the oracle consumes comes from the GPU path except
the outputs being checked."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from compressed_sparse_attention_07_amd import csa2 as C
from compressed_sparse_attention_07_amd import synth

DEV = "cuda"
ATT_TOL = 2e-3  # max |O - O*| <= 2e-3 * max |V attended|


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def seqs_for(lengths, row0s, cache_rows) -> C.Seqs:
    lengths = np.asarray(lengths, dtype=np.int64)
    return C.Seqs(
        kv_row0=torch.tensor(np.asarray(row0s, dtype=np.int64), device=DEV),
        kv_len=torch.tensor(lengths.astype(np.int32), device=DEV),
        max_len_ub=int(lengths.max()) if lengths.size else 0,
        total_len_ub=int(lengths.sum()),
        cache_rows=int(cache_rows),
    )


def packed_rows(lengths):
    """Row offsets for sequences stored back to back."""
    lengths = np.asarray(lengths, dtype=np.int64)
    row0 = np.zeros_like(lengths)
    row0[1:] = np.cumsum(lengths)[:-1]
    return row0, int(lengths.sum())


class IndexCase:
    """Integer-valued indexer inputs for ragged sequences stored back to back."""

    def __init__(self, workload, lengths, n_heads=4, kfill=None, qlo=-4, qhi=4, seed=0):
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.row0, rows = packed_rows(self.lengths)
        self.rows = max(rows, 1)
        n_q = len(lengths)
        if kfill is None:
            self.k = synth.int_bf16(workload, synth.T_IDX_K, (self.rows, 64), qlo, qhi, seq=seed)
        else:
            self.k = np.full((self.rows, 64), kfill, dtype=np.uint16)
        self.q = synth.int_bf16(workload, synth.T_IDX_Q, (n_q, n_heads, 64), qlo, qhi, seq=seed)
        self.w = synth.int_weights(workload, synth.T_IDX_W, (n_q, n_heads), seq=seed)
        self.n_heads = n_heads
        self.k_dev = bf16_tensor(self.k)
        self.q_dev = bf16_tensor(self.q)
        self.w_dev = torch.from_numpy(self.w).to(DEV)
        self.seqs = seqs_for(self.lengths, self.row0, self.rows)

    def oracle_full(self, i, top_k, pool_blocks):
        r0, n = int(self.row0[i]), int(self.lengths[i])
        return O.index_full(self.q[i], self.w[i], self.k[r0:r0 + max(n, 0)], n, top_k, 8, pool_blocks)

    def oracle_reindex(self, i, pool, top_k, q=None, w=None):
        r0, n = int(self.row0[i]), int(self.lengths[i])
        q = self.q[i] if q is None else q
        w = self.w[i] if w is None else w
        return O.index_reindex(q, w, self.k[r0:r0 + max(n, 0)], n, pool, top_k, 8)

    def run_full(self, top_k, pool_blocks, ws=None, shared_kv=0):
        n_q = len(self.lengths)
        need = C.csa2_workspace_bytes(C.OP_INDEX_FULL, n_q, self.seqs.total_len_ub, self.seqs.max_len_ub, top_k,
                                      pool_blocks)
        assert 0 < need < C.SIZE_MAX
        ws = ws if ws is not None else C.alloc_workspace(need)
        idx = torch.full((n_q, top_k), -7, dtype=torch.int32, device=DEV)
        pool = torch.full((n_q, max(pool_blocks, 1)), -7, dtype=torch.int32, device=DEV) if pool_blocks else None
        C.csa2_index_full(self.q_dev, self.w_dev, self.k_dev, self.seqs, top_k, pool_blocks, idx, pool, ws,
                          shared_kv=shared_kv)
        torch.cuda.synchronize()
        return idx, pool, ws

    def run_reindex(self, pool, top_k, q_dev=None, w_dev=None, ws=None):
        n_q = len(self.lengths)
        need = C.csa2_workspace_bytes(C.OP_INDEX_REINDEX, n_q, 0, 0, top_k, pool.shape[1])
        ws = ws if ws is not None else C.alloc_workspace(need)
        idx = torch.full((n_q, top_k), -7, dtype=torch.int32, device=DEV)
        C.csa2_index_reindex(self.q_dev if q_dev is None else q_dev, self.w_dev if w_dev is None else w_dev,
                             self.k_dev, self.seqs, pool, top_k, idx, ws)
        torch.cuda.synchronize()
        return idx, ws


class SharedIndexCase(IndexCase):
    """Queries that all read one sequence (a prefill chunk): query t sees lengths[t] positions."""

    def __init__(self, workload, rows, lengths, n_heads=4, qlo=-4, qhi=4, seed=0):
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.row0 = np.zeros(len(lengths), dtype=np.int64)
        self.rows = rows
        n_q = len(lengths)
        self.k = synth.int_bf16(workload, synth.T_IDX_K, (rows, 64), qlo, qhi, seq=seed)
        self.q = synth.int_bf16(workload, synth.T_IDX_Q, (n_q, n_heads, 64), qlo, qhi, seq=seed)
        self.w = synth.int_weights(workload, synth.T_IDX_W, (n_q, n_heads), seq=seed)
        self.n_heads = n_heads
        self.k_dev = bf16_tensor(self.k)
        self.q_dev = bf16_tensor(self.q)
        self.w_dev = torch.from_numpy(self.w).to(DEV)
        self.seqs = seqs_for(self.lengths, self.row0, rows)


class AttendCase:
    """FP4 cache (packed by the GPU path and checked bit-exact against the oracle first),
    a per-query bf16 window ring, and queries."""

    def __init__(self, workload, lengths, n_heads=16, window=128, swa_cap=128, seed=0):
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.row0, rows = packed_rows(self.lengths)
        self.rows = max(rows, 1)
        n_q = len(lengths)
        sig = synth.channel_sigma(workload, synth.T_KV_SIGMA, 128, seq=seed)
        self.x = synth.kv_bf16(workload, synth.T_KV, self.rows, 128, sig, seq=seed)
        self.codes_ref, self.scales_ref = O.fp4_quantize(self.x)
        self.codes = torch.zeros((self.rows, 64), dtype=torch.uint8, device=DEV)
        self.scales = torch.zeros((self.rows, 8), dtype=torch.uint8, device=DEV)
        C.fp4_kv_append(bf16_tensor(self.x), self.codes, self.scales)
        torch.cuda.synchronize()
        assert np.array_equal(self.codes.cpu().numpy(), self.codes_ref)
        assert np.array_equal(self.scales.cpu().numpy(), self.scales_ref)
        ssig = synth.channel_sigma(workload, synth.T_SWA_SIGMA, 128, seq=seed)
        self.swa_cap = swa_cap
        self.swa = synth.kv_bf16(workload, synth.T_SWA, n_q * swa_cap, 128, ssig, seq=seed)
        self.swa_row0 = np.arange(n_q, dtype=np.int64) * swa_cap
        self.window = window
        self.q = synth.normal_bf16(workload, synth.T_Q, (n_q, n_heads, 128), seq=seed)
        self.n_heads = n_heads
        self.seqs = seqs_for(self.lengths, self.row0, self.rows)
        self.swa_dev = bf16_tensor(self.swa)
        self.swa_row0_dev = torch.from_numpy(self.swa_row0).to(DEV)
        self.q_dev = bf16_tensor(self.q)

    def run(self, idx_np: np.ndarray, scale: float, ws=None):
        n_q = len(self.lengths)
        top_k = idx_np.shape[1]
        need = C.csa2_workspace_bytes(C.OP_ATTEND, n_q, 0, 0, top_k, self.window)
        ws = ws if ws is not None else C.alloc_workspace(need)
        out = torch.full((n_q, self.n_heads, 128), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.from_numpy(np.ascontiguousarray(idx_np.astype(np.int32))).to(DEV)
        C.csa2_attend(self.q_dev, self.codes, self.scales, self.seqs, idx, self.swa_dev, self.swa_row0_dev,
                      self.swa_cap, self.window, scale, out, ws=ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), ws

    def check(self, out, idx_np, scale, i_list=None):
        worst = 0.0
        for i in (range(len(self.lengths)) if i_list is None else i_list):
            r0, n = int(self.row0[i]), int(self.lengths[i])
            ref = O.attend(self.q[i], self.codes_ref[r0:r0 + n], self.scales_ref[r0:r0 + n], n, idx_np[i],
                           self.swa, int(self.swa_row0[i]), self.swa_cap, self.window, scale)
            vmax = O.attended_max_abs(self.codes_ref[r0:r0 + n], self.scales_ref[r0:r0 + n], n, idx_np[i],
                                      self.swa, int(self.swa_row0[i]), self.swa_cap, self.window)
            err = float(np.abs(out[i].astype(np.float64) - ref).max())
            if vmax == 0.0:
                assert err == 0.0, (i, err)
            else:
                assert err <= ATT_TOL * vmax, (i, err, vmax)
                worst = max(worst, err / vmax)
        return worst
