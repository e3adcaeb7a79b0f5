"""GPU parity of each entry point against the CPU oracle at small and ragged sizes:
bit-exact FP4 codes, scales, Top-K indices and pools; attention within 2e-3 * max|V|."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_attention_07_amd import csa2 as C
from compressed_sparse_attention_07_amd import synth

from gpu_helpers import AttendCase, IndexCase, SharedIndexCase, bf16_tensor, DEV

pytestmark = pytest.mark.gpu

W_T = 900  # workload id for these tests' seeds


# ---------------------------------------------------------------- FP4 pack-on-write
@pytest.mark.parametrize("n_tok,dim", [(1, 128), (7, 16), (1000, 128), (4099, 128), (333, 1024), (64, 48)])
def test_fp4_pack_bit_exact(n_tok, dim):
    sig = synth.channel_sigma(W_T, synth.T_KV_SIGMA, dim, seq=n_tok)
    x = synth.kv_bf16(W_T, synth.T_KV, n_tok, dim, sig, seq=n_tok)
    codes = torch.zeros((n_tok, dim // 2), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((n_tok, dim // 16), dtype=torch.uint8, device=DEV)
    C.fp4_kv_append(bf16_tensor(x), codes, scales)
    c_ref, s_ref = O.fp4_quantize(x)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(scales.cpu().numpy(), s_ref)


def _special_groups():
    f = synth.f32_to_bf16_bits
    rows = []
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for s in [1.0, 2.0 ** -9, 2.0 ** -6, 0.4375, 4.5, 448.0]:
        g = [6 * s] + [m * s for m in mids] + [-m * s for m in mids] + [0.0]
        rows.append(f(np.array(g, np.float32)))
    rows.append(np.zeros(16, np.uint16))                    # amax 0
    rows.append(np.full(16, 0x8000, np.uint16))             # all -0
    rows.append(f(np.array([6 * 2.0 ** -10] + [0.0] * 15, np.float32)))   # scale tie to 0
    rows.append(f(np.array([6.375] + [-6.375] * 15, np.float32)))         # saturation
    rows.append(f(np.array([2688.0, -2688.0, 1.0] + [0.0] * 13, np.float32)))
    r = np.random.default_rng(5)
    for _ in range(200):                                     # every bf16 pattern class
        rows.append(r.integers(0, 0x7F80, 16).astype(np.uint16) | (r.integers(0, 2, 16).astype(np.uint16) << 15))
    x = np.stack(rows)
    # keep finite, |x| <= 2688
    v = O.bf16_to_f64(x)
    x[np.abs(v) > 2688] = 0
    return x


def test_fp4_pack_every_scale_and_midpoint():
    # For every E4M3 scale code c (1..126): groups whose largest element is exactly 6 v(c), so
    # the scale is c, and whose other 15 elements sit on the E2M1 midpoints m v(c) (exact ties)
    # and one bf16 step to either side, in even and odd channels, with both signs -- every
    # rounding decision of the packer at every scale, compared with the oracle.
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows = []
    rng = np.random.default_rng(17)
    for c in range(1, 127):
        e, m = c >> 3, c & 7
        v = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8)
        vals = []
        for mid in mids:
            b = int(np.float32(mid * v).view(np.uint32)) >> 16           # exact bf16 threshold
            vals += [b, b + 1, b - 1]
        top = int(np.float32(6 * v).view(np.uint32)) >> 16
        for shift in range(2):                                          # odd / even placement
            vv = np.array(vals, dtype=np.int64)
            rng.shuffle(vv)
            for start in range(0, len(vv), 15):
                chunk = list(vv[start:start + 15])
                chunk += [0] * (15 - len(chunk))
                g = chunk[:shift] + [top] + chunk[shift:]
                sign = rng.integers(0, 2, 16) << 15
                rows.append((np.array(g, dtype=np.int64) | sign).astype(np.uint16))
    x = np.stack(rows)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 8, 16), np.uint16)]).reshape(-1, 128)
    codes = torch.full((x.shape[0], 64), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((x.shape[0], 8), 0x5A, dtype=torch.uint8, device=DEV)
    C.fp4_kv_append(bf16_tensor(x), codes, scales)
    torch.cuda.synchronize()
    c_ref, s_ref = O.fp4_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


def test_fp4_pack_special_groups():
    x = _special_groups()
    x = np.concatenate([x] * 8, axis=1)[:, :128]             # 128 channels per row
    n = x.shape[0]
    codes = torch.zeros((n, 64), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((n, 8), dtype=torch.uint8, device=DEV)
    C.fp4_kv_append(bf16_tensor(x), codes, scales)
    c_ref, s_ref = O.fp4_quantize(x)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


def test_fp4_pack_scatter_rows_and_skips_out_of_range():
    n_tok, cap = 50, 80
    sig = synth.channel_sigma(W_T, synth.T_KV_SIGMA, 128, seq=77)
    x = synth.kv_bf16(W_T, synth.T_KV, n_tok, 128, sig, seq=77)
    rows = np.random.default_rng(3).permutation(cap)[:n_tok].astype(np.int64)
    rows[5] = -1
    rows[9] = cap + 3
    codes = torch.full((cap, 64), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((cap, 8), 0xCD, dtype=torch.uint8, device=DEV)
    C.fp4_kv_append(bf16_tensor(x), codes, scales, dst_rows=torch.from_numpy(rows).to(DEV))
    c_ref, s_ref = O.fp4_quantize(x)
    cg, sg = codes.cpu().numpy(), scales.cpu().numpy()
    written = set()
    for t, r in enumerate(rows):
        if 0 <= r < cap:
            assert np.array_equal(cg[r], c_ref[t]) and np.array_equal(sg[r], s_ref[t])
            written.add(int(r))
    for r in range(cap):
        if r not in written:
            assert np.all(cg[r] == 0xAB) and np.all(sg[r] == 0xCD)


@pytest.mark.parametrize("mx", [False, True])
def test_token_append_kv_and_key_rows(mx):
    # the decode step's own token of a Full layer's set: FP4 KV row (as fp4_kv_append) and its
    # indexer key row (a bf16 copy, or MXFP4 as mxfp4_key_append) in one launch; rows outside
    # the cache are skipped and every other row is left alone
    n, cap = 37, 300
    x = synth.kv_bf16(W_T + 7, synth.T_NEW_KV, n, 128, synth.channel_sigma(W_T + 7, synth.T_KV_SIGMA, 128))
    k = synth.int_bf16(W_T + 7, synth.T_IDX_K, (n, 64), seq=1)
    rows = np.random.default_rng(7).permutation(cap)[:n].astype(np.int64)
    rows[3], rows[11] = -1, cap + 5
    codes = torch.full((cap, 64), 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full((cap, 8), 0x5A, dtype=torch.uint8, device=DEV)
    if mx:
        kc = torch.full((cap, 32), 0x5A, dtype=torch.uint8, device=DEV)
        ks = torch.full((cap, 2), 0x5A, dtype=torch.uint8, device=DEV)
        C.csa2_token_append(bf16_tensor(x), torch.from_numpy(rows).to(DEV), codes, scales, k_new=bf16_tensor(k),
                            k_idx=kc, k_scales=ks)
    else:
        kb = torch.full((cap, 64), 0x5A5A, dtype=torch.int16, device=DEV)
        C.csa2_token_append(bf16_tensor(x), torch.from_numpy(rows).to(DEV), codes, scales, k_new=bf16_tensor(k),
                            k_idx=kb)
    torch.cuda.synchronize()
    c_ref, s_ref = O.fp4_quantize(x)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    ok = (rows >= 0) & (rows < cap)
    assert np.array_equal(got_c[rows[ok]], c_ref[ok]) and np.array_equal(got_s[rows[ok]], s_ref[ok])
    untouched = np.setdiff1d(np.arange(cap), rows[ok])
    assert (got_c[untouched] == 0x5A).all() and (got_s[untouched] == 0x5A).all()
    if mx:
        kc_ref, ks_ref = O.mxfp4_quantize(k)
        assert np.array_equal(kc.cpu().numpy()[rows[ok]], kc_ref[ok])
        assert np.array_equal(ks.cpu().numpy()[rows[ok]], ks_ref[ok])
        assert (kc.cpu().numpy()[untouched] == 0x5A).all()
    else:
        got_k = kb.cpu().numpy().view(np.uint16)
        assert np.array_equal(got_k[rows[ok]], k[ok])
        assert (got_k[untouched] == 0x5A5A).all()


@pytest.mark.parametrize("fp8", [False, True])
def test_window_append_rows(fp8):
    x = synth.kv_bf16(W_T + 8, synth.T_SWA, 50, 128, synth.channel_sigma(W_T + 8, synth.T_SWA_SIGMA, 128))
    rows = np.arange(50, dtype=np.int64)[::-1].copy() * 2
    rows[0] = 1000                                              # outside: skipped
    store = torch.zeros((100, 128), dtype=torch.uint8 if fp8 else torch.int16, device=DEV)
    C.csa2_window_append(bf16_tensor(x), store, dst_rows=torch.from_numpy(rows).to(DEV), window_fp8=fp8)
    torch.cuda.synchronize()
    got = store.cpu().numpy()
    want = O.e4m3_quantize(x) if fp8 else x
    got = got if fp8 else got.view(np.uint16)
    assert np.array_equal(got[rows[1:]], want[1:])
    assert (got[1::2] == 0).all()


def test_fp4_pack_row_offset_appends():
    sig = synth.channel_sigma(W_T, synth.T_KV_SIGMA, 128, seq=78)
    x = synth.kv_bf16(W_T, synth.T_KV, 10, 128, sig, seq=78)
    codes = torch.zeros((30, 64), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((30, 8), dtype=torch.uint8, device=DEV)
    C.fp4_kv_append(bf16_tensor(x), codes, scales, row0=17)
    c_ref, s_ref = O.fp4_quantize(x)
    assert np.array_equal(codes.cpu().numpy()[17:27], c_ref)
    assert np.all(codes.cpu().numpy()[:17] == 0) and np.all(codes.cpu().numpy()[27:] == 0)
    with pytest.raises(C.Csa2Error):
        C.fp4_kv_append(bf16_tensor(x), codes, scales, row0=25)


# ---------------------------------------------------------------- Full mode
RAGGED = [0, 1, 7, 8, 9, 511, 512, 513, 2047, 2048, 2049, 4101, 20000]


@pytest.mark.parametrize("top_k,pool_blocks,n_heads", [(512, 256, 4), (3, 1, 1), (64, 5, 8), (1, 0, 3),
                                                       (2048, 2048, 4)])
def test_index_full_bit_exact_ragged(top_k, pool_blocks, n_heads):
    case = IndexCase(W_T + top_k, RAGGED, n_heads=n_heads)
    idx, pool, _ = case.run_full(top_k, pool_blocks)
    idx = idx.cpu().numpy()
    pool = pool.cpu().numpy() if pool is not None else None
    for i in range(len(RAGGED)):
        ri, rp = case.oracle_full(i, top_k, pool_blocks)
        assert np.array_equal(idx[i], ri), (i, RAGGED[i])
        if pool_blocks:
            assert np.array_equal(pool[i], rp), (i, RAGGED[i])


# every context <= 16,384: the selection workgroups split the keys themselves (no filter kernel)
RAGGED_SHORT = [0, 1, 7, 8, 9, 511, 512, 513, 2047, 2048, 2049, 4101, 16383, 16384]


@pytest.mark.parametrize("top_k,pool_blocks,n_heads", [(512, 256, 4), (2048, 2048, 4), (3, 1, 1)])
def test_index_full_bit_exact_short_contexts(top_k, pool_blocks, n_heads):
    case = IndexCase(W_T + 70 + top_k, RAGGED_SHORT, n_heads=n_heads)
    idx, pool, _ = case.run_full(top_k, pool_blocks)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for i in range(len(RAGGED_SHORT)):
        ri, rp = case.oracle_full(i, top_k, pool_blocks)
        assert np.array_equal(idx[i], ri), (i, RAGGED_SHORT[i])
        assert np.array_equal(pool[i], rp), (i, RAGGED_SHORT[i])


def test_index_full_tie_heavy_short_contexts():
    lengths = [3000, 16384, 12345, 5]
    case = IndexCase(W_T + 71, lengths, n_heads=4, qlo=0, qhi=1)   # scores in a narrow integer range
    idx, pool, _ = case.run_full(512, 700)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for i in range(len(lengths)):
        ri, rp = case.oracle_full(i, 512, 700)
        assert np.array_equal(idx[i], ri), i
        assert np.array_equal(pool[i], rp), i


def test_index_full_many_queries():
    # more queries than one workgroup's scan width: the ragged tile map is built in chunks
    lengths = list(np.random.default_rng(21).integers(0, 5000, size=300))
    case = IndexCase(W_T + 9, lengths, n_heads=4)
    idx, pool, _ = case.run_full(16, 8)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for i in range(0, 300, 7):
        ri, rp = case.oracle_full(i, 16, 8)
        assert np.array_equal(idx[i], ri), i
        assert np.array_equal(pool[i], rp), i


def test_index_full_more_queries_than_one_prep_chunk():
    # 1,300 decode queries: the metadata kernel handles them in chunks of 1,024 (tile runs carried
    # across chunks), with every context short enough for the filter-free selection
    lengths = list(np.random.default_rng(23).integers(0, 2500, size=1300))
    case = IndexCase(W_T + 11, lengths, n_heads=4)
    idx, pool, _ = case.run_full(64, 16)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for i in list(range(0, 1300, 13)) + [1023, 1024, 1025, 1299]:
        ri, rp = case.oracle_full(i, 64, 16)
        assert np.array_equal(idx[i], ri), i
        assert np.array_equal(pool[i], rp), i


@pytest.mark.parametrize("n_q", [64, 65])
def test_index_full_one_wave_of_queries_and_one_more(n_q):
    # 64 decode queries: the scan derives the tile runs itself and writes the metadata and the
    # filter map the later kernels read; 65: the metadata kernel does.  Both bit-exact, with
    # empty, single-tile and many-filter-tile contexts in one call.
    rng = np.random.default_rng(27 + n_q)
    lengths = [int(x) for x in rng.integers(0, 9000, size=n_q)]
    lengths[0], lengths[5], lengths[31], lengths[n_q - 1] = 0, 41000, 0, 70001
    case = IndexCase(W_T + 13 + n_q, lengths, n_heads=4)
    idx, pool, _ = case.run_full(512, 300)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for i in sorted({0, 1, 5, 30, 31, 32, 62, 63, n_q - 1} | set(range(0, n_q, 9))):
        ri, rp = case.oracle_full(i, 512, 300)
        assert np.array_equal(idx[i], ri), (n_q, i, lengths[i])
        assert np.array_equal(pool[i], rp), (n_q, i, lengths[i])


def test_index_full_timed_scan_equals_single_call():
    # prep -> timed scan (the kernel records its start and end into two events) -> select gives
    # exactly the single call's selection, and the events bracket a positive interval
    lengths = [70000, 20000, 4096, 0, 9]
    case = IndexCase(W_T + 12, lengths, n_heads=4)
    idx_ref, pool_ref, _ = case.run_full(512, 300)
    n_q = len(lengths)
    ws = C.alloc_workspace(C.csa2_workspace_bytes(C.OP_INDEX_FULL, n_q, case.seqs.total_len_ub,
                                                  case.seqs.max_len_ub, 512, 300))
    idx = torch.full((n_q, 512), -7, dtype=torch.int32, device=DEV)
    pool = torch.full((n_q, 300), -7, dtype=torch.int32, device=DEV)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    C.csa2_index_full_prep(case.q_dev, case.w_dev, case.k_dev, case.seqs, 512, 300, idx, pool, ws)
    C.csa2_index_full_scan_timed(case.q_dev, case.w_dev, case.k_dev, None, case.seqs, 512, 300, idx, pool, ws, e0, e1)
    C.csa2_index_full_select(case.q_dev, case.w_dev, case.k_dev, case.seqs, 512, 300, idx, pool, ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_ref) and torch.equal(pool, pool_ref)
    assert e0.elapsed_time(e1) > 0.0


def test_index_full_tie_heavy_and_repeatable():
    lengths = [3000, 70000, 12345]
    case = IndexCase(W_T + 1, lengths, n_heads=4, qlo=0, qhi=1)   # scores in a narrow integer range
    ws = None
    first = None
    for rep in range(3):                                            # the workspace cleans itself
        idx, pool, ws = case.run_full(512, 700, ws=ws)
        got = (idx.cpu().numpy(), pool.cpu().numpy())
        if first is None:
            first = got
        else:
            assert np.array_equal(got[0], first[0]) and np.array_equal(got[1], first[1])
    for i in range(len(lengths)):
        ri, rp = case.oracle_full(i, 512, 700)
        assert np.array_equal(first[0][i], ri)
        assert np.array_equal(first[1][i], rp)


@pytest.mark.parametrize("lengths,pool_blocks", [([50000, 9000], 2048), ([5000, 800, 513], 50),
                                                 ([12000, 16384, 600], 2048)])
def test_index_full_all_equal_scores_takes_lowest_positions(lengths, pool_blocks):
    # every score is 0: the whole context is one tie band.  50,000 / 9,000: larger than the LDS
    # candidate set; 5,000 / 1,125 blocks: in LDS with more ties than are ordered directly;
    # 800 / 513 positions and 100 / 65 blocks: ties ordered directly by position; 12,000 and
    # 16,384 (contexts the selection workgroup splits itself): larger than the LDS set
    case = IndexCase(W_T + 2, lengths, n_heads=4, kfill=0)
    idx, pool, _ = case.run_full(512, pool_blocks)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for i in range(len(lengths)):
        assert np.array_equal(idx[i], np.arange(512))
        nb = -(-lengths[i] // 8)
        assert np.array_equal(pool[i], np.arange(pool_blocks) if nb >= pool_blocks else
                              np.concatenate([np.arange(nb), -np.ones(pool_blocks - nb, int)]))


# ---------------------------------------------------------------- prefill chunk (MFMA scoring)
@pytest.mark.parametrize("n_heads,top_k", [(4, 512), (3, 100), (1, 7)])
def test_index_prefill_mfma_causal_bit_exact(n_heads, top_k):
    # 100 queries of one 6,000-position sequence; query t sees C + t + 1 positions
    C_, T = 5900, 100
    case = SharedIndexCase(W_T + 40 + n_heads, C_ + T, C_ + 1 + np.arange(T), n_heads=n_heads)
    idx_m, _, _ = case.run_full(top_k, 0, shared_kv=1)
    idx_v, _, _ = case.run_full(top_k, 0, shared_kv=0)          # per-query decode path on the same data
    idx_m, idx_v = idx_m.cpu().numpy(), idx_v.cpu().numpy()
    assert np.array_equal(idx_m, idx_v)
    for t in list(range(0, T, 9)) + [T - 1]:
        ri, _ = case.oracle_full(t, top_k, 0)
        assert np.array_equal(idx_m[t], ri), t


def test_index_prefill_mfma_arbitrary_lengths_and_ties():
    # lengths in any order (not monotone), including empty and tiny queries, tie-heavy scores
    lengths = [0, 1, 17, 4096, 4097, 9000, 3, 12345, 8191, 8192, 8193, 50, 7777, 2, 1000, 6000, 12000, 5]
    case = SharedIndexCase(W_T + 50, 12345, lengths, n_heads=4, qlo=0, qhi=1)
    idx_m, _, _ = case.run_full(512, 0, shared_kv=1)
    idx_m = idx_m.cpu().numpy()
    for t in range(len(lengths)):
        ri, _ = case.oracle_full(t, 512, 0)
        assert np.array_equal(idx_m[t], ri), t


@pytest.mark.parametrize("pool_blocks", [300, 1, 2048])
def test_index_prefill_mfma_per_query_pools(pool_blocks):
    # a prefill chunk with pools: every query token gets the pool of its own visible positions
    # (partial last blocks included), bit-exact against the oracle and the per-query decode path;
    # then a Reindex layer over those per-query pools
    lengths = [0, 1, 9, 4096, 4097, 9000, 3, 12345, 8191, 8192, 8193, 50, 7777, 2, 1000, 6000, 12000, 5]
    case = SharedIndexCase(W_T + 60, 12345, lengths, n_heads=4)
    idx_m, pool_m, _ = case.run_full(512, pool_blocks, shared_kv=1)
    idx_v, pool_v, _ = case.run_full(512, pool_blocks, shared_kv=0)
    idx_m, pool_m = idx_m.cpu().numpy(), pool_m.cpu().numpy()
    assert np.array_equal(idx_m, idx_v.cpu().numpy()) and np.array_equal(pool_m, pool_v.cpu().numpy())
    for t in range(len(lengths)):
        ri, rp = case.oracle_full(t, 512, pool_blocks)
        assert np.array_equal(idx_m[t], ri), t
        assert np.array_equal(pool_m[t], rp), t
    q2 = synth.int_bf16(W_T + 60, synth.T_IDX_Q, (len(lengths), 4, 64), seq=3)
    w2 = synth.int_weights(W_T + 60, synth.T_IDX_W, (len(lengths), 4), seq=3)
    idx2, _ = case.run_reindex(torch.from_numpy(pool_m).to(DEV), 512, q_dev=bf16_tensor(q2),
                               w_dev=torch.from_numpy(w2).to(DEV))
    idx2 = idx2.cpu().numpy()
    for t in range(len(lengths)):
        assert np.array_equal(idx2[t], case.oracle_reindex(t, pool_m[t], 512, q=q2[t], w=w2[t])), t


def test_index_prefill_fractional_and_negative_weights():
    # the prefill scoring passes build the key from the score without the -0 step (a sum started
    # from +0 is never -0): scores of both signs with bits below the integer part, exact in fp32
    C_, T = 9000, 48
    case = SharedIndexCase(W_T + 83, C_ + T, C_ + 1 + np.arange(T), n_heads=4)
    m = np.random.default_rng(83).integers(-256, 257, size=case.w.shape)
    m[m == 0] = 3
    case.w = (m / 64.0).astype(np.float32)
    case.w_dev = torch.from_numpy(case.w).to(DEV)
    idx_m, pool_m, _ = case.run_full(512, 300, shared_kv=1)
    idx_m, pool_m = idx_m.cpu().numpy(), pool_m.cpu().numpy()
    for t in range(T):
        ri, rp = case.oracle_full(t, 512, 300)
        assert np.array_equal(idx_m[t], ri), t
        assert np.array_equal(pool_m[t], rp), t


def test_index_prefill_all_negative_weights():
    # every score <= 0: the sample's threshold falls among negative scores, which its histogram
    # counts as digit 0, so every visible position becomes a candidate; still bit-exact
    C_, T = 9000, 48
    case = SharedIndexCase(W_T + 84, C_ + T, C_ + 1 + np.arange(T), n_heads=4)
    m = np.random.default_rng(84).integers(1, 257, size=case.w.shape)
    case.w = (-m / 64.0).astype(np.float32)
    case.w_dev = torch.from_numpy(case.w).to(DEV)
    idx_m, pool_m, _ = case.run_full(512, 300, shared_kv=1)
    idx_m, pool_m = idx_m.cpu().numpy(), pool_m.cpu().numpy()
    for t in range(T):
        ri, rp = case.oracle_full(t, 512, 300)
        assert np.array_equal(idx_m[t], ri), t
        assert np.array_equal(pool_m[t], rp), t


def test_index_reindex_many_queries_whole_pool_per_workgroup():
    # >= 512 queries with 2,048-block pools: each Reindex workgroup scores a whole pool and adds
    # its counts to the query's histogram once; every token checked against the oracle
    T = 600
    lengths = np.random.default_rng(90).integers(1, 20000, size=T)
    case = SharedIndexCase(W_T + 90, 20000, lengths, n_heads=4)
    _, pool, _ = case.run_full(512, 2048, shared_kv=1)
    q2 = synth.int_bf16(W_T + 90, synth.T_IDX_Q, (T, 4, 64), seq=7)
    w2 = synth.int_weights(W_T + 90, synth.T_IDX_W, (T, 4), seq=7)
    idx2, _ = case.run_reindex(pool, 512, q_dev=bf16_tensor(q2), w_dev=torch.from_numpy(w2).to(DEV))
    idx2, pool_np = idx2.cpu().numpy(), pool.cpu().numpy()
    for t in range(T):
        assert np.array_equal(idx2[t], case.oracle_reindex(t, pool_np[t], 512, q=q2[t], w=w2[t])), t


@pytest.mark.parametrize("tokens", [32, 600])
def test_index_prefill_all_equal_scores_takes_lowest_positions(tokens):
    # every score is 0: every visible position of every token is in the threshold bucket, so
    # the compacting pass overflows its per-token LDS buffer and writes the rest directly; with
    # 600 tokens the selection runs its many-query form, whose LDS holds 2,048 candidates, so
    # these buckets (3,000+ positions) take its global-list path
    lengths = [3000 + 7 * (t % 40) for t in range(tokens)]
    case = SharedIndexCase(W_T + 62, 3300, lengths, n_heads=4, qlo=0, qhi=0)
    idx, pool, _ = case.run_full(512, 100, shared_kv=1)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for t in range(len(lengths)):
        assert np.array_equal(idx[t], np.arange(512)), t
        assert np.array_equal(pool[t], np.arange(100)), t


def test_index_prefill_nothing_visible():
    # a chunk of 16 queries that see no position at all: every output is -1 padding
    case = SharedIndexCase(W_T + 61, 64, [0] * 16, n_heads=4)
    idx, pool, _ = case.run_full(512, 300, shared_kv=1)
    assert (idx.cpu().numpy() == -1).all() and (pool.cpu().numpy() == -1).all()


# ---------------------------------------------------------------- Reindex mode
def test_index_reindex_bit_exact_and_invariant():
    lengths = [4096, 65536, 777, 100, 30001]
    case = IndexCase(W_T + 3, lengths, n_heads=4)
    idx_f, pool, _ = case.run_full(512, 2048)
    # Reindex with the Full layer's own query returns the Full Top-K (K <= P)
    idx_r, _ = case.run_reindex(pool, 512)
    assert np.array_equal(idx_r.cpu().numpy(), idx_f.cpu().numpy())
    # another layer's query: bit-exact against the oracle
    q2 = synth.int_bf16(W_T + 3, synth.T_IDX_Q, (len(lengths), 4, 64), seq=9)
    w2 = synth.int_weights(W_T + 3, synth.T_IDX_W, (len(lengths), 4), seq=9)
    idx2, _ = case.run_reindex(pool, 512, q_dev=bf16_tensor(q2), w_dev=torch.from_numpy(w2).to(DEV))
    idx2 = idx2.cpu().numpy()
    pool_np = pool.cpu().numpy()
    for i in range(len(lengths)):
        ref = case.oracle_reindex(i, pool_np[i], 512, q=q2[i], w=w2[i])
        assert np.array_equal(idx2[i], ref), i


@pytest.mark.parametrize("negative", [False, True])
def test_index_fractional_weights_full_and_reindex(negative):
    # weights m / 64 (|m| <= 256): every score is still exact in fp32 and fp64 (at most 20
    # significant bits), but keys now carry bits below the integer part, so the radix passes
    # cannot stop early on all-zero low bits; negative weights give negative scores (keys with
    # every bit flipped)
    lengths = [70000, 20000, 4096, 9]
    case = IndexCase(W_T + 80 + int(negative), lengths, n_heads=4)
    r = np.random.default_rng(80 + int(negative))
    lo = -256 if negative else 1
    m = r.integers(lo, 257, size=case.w.shape)
    m[m == 0] = 1
    case.w = (m / 64.0).astype(np.float32)
    case.w_dev = torch.from_numpy(case.w).to(DEV)
    idx_f, pool, _ = case.run_full(512, 2048)
    idx_f, pool_np = idx_f.cpu().numpy(), pool.cpu().numpy()
    for i in range(len(lengths)):
        ri, rp = case.oracle_full(i, 512, 2048)
        assert np.array_equal(idx_f[i], ri), i
        assert np.array_equal(pool_np[i], rp), i
    q2 = synth.int_bf16(W_T + 82, synth.T_IDX_Q, (len(lengths), 4, 64), seq=5)
    w2 = (r.integers(lo, 257, size=(len(lengths), 4)) / 64.0).astype(np.float32)
    w2[w2 == 0] = 1.0
    idx2, _ = case.run_reindex(pool, 512, q_dev=bf16_tensor(q2), w_dev=torch.from_numpy(w2).to(DEV))
    idx2 = idx2.cpu().numpy()
    for i in range(len(lengths)):
        assert np.array_equal(idx2[i], case.oracle_reindex(i, pool_np[i], 512, q=q2[i], w=w2[i])), i


@pytest.mark.parametrize("n_q,n_heads", [(16, 4), (17, 4), (16, 8)])
def test_index_reindex_lane_per_position_and_row_forms(n_q, n_heads):
    # up to 16 queries with at most 4 heads score one position per lane; 17 queries, or 8 heads,
    # take the 16-position form: both against the oracle on ragged contexts (pools with padding)
    lengths = np.random.default_rng(95 + n_q).integers(1, 40000, size=n_q)
    lengths[0], lengths[-1] = 9, 16384
    case = IndexCase(W_T + 95 + n_q, lengths, n_heads=n_heads)
    _, pool, _ = case.run_full(512, 2048)
    q2 = synth.int_bf16(W_T + 95, synth.T_IDX_Q, (n_q, n_heads, 64), seq=11)
    w2 = synth.int_weights(W_T + 95, synth.T_IDX_W, (n_q, n_heads), seq=11)
    idx2, _ = case.run_reindex(pool, 512, q_dev=bf16_tensor(q2), w_dev=torch.from_numpy(w2).to(DEV))
    idx2, pool_np = idx2.cpu().numpy(), pool.cpu().numpy()
    for i in range(n_q):
        assert np.array_equal(idx2[i], case.oracle_reindex(i, pool_np[i], 512, q=q2[i], w=w2[i])), i


@pytest.mark.parametrize("top_k,pool_blocks", [(1024, 1024), (1025, 1025)])
def test_index_prefill_selection_sizes_around_lds_lists(top_k, pool_blocks):
    # 512 queries of one chunk: selections of at most 1,024 entries are gathered in LDS lists of
    # that size, larger ones in the 2,048-entry form; both sides of the limit, for the position
    # list and the pool list, every query against the oracle
    T = 512
    lengths = np.random.default_rng(96).integers(1, 12000, size=T)
    lengths[:4] = [8200, 8192, 1024, 3]
    case = SharedIndexCase(W_T + 96, 12000, lengths, n_heads=4)
    idx, pool, _ = case.run_full(top_k, pool_blocks, shared_kv=1)
    idx, pool = idx.cpu().numpy(), pool.cpu().numpy()
    for t in range(T):
        ri, rp = case.oracle_full(t, top_k, pool_blocks)
        assert np.array_equal(idx[t], ri), t
        assert np.array_equal(pool[t], rp), t


def test_index_reindex_pool_with_padding_and_out_of_range_blocks():
    lengths = [1000, 50]
    case = IndexCase(W_T + 4, lengths, n_heads=4)
    pool = np.full((2, 40), -1, dtype=np.int32)
    pool[0, :10] = np.arange(0, 100, 10)
    pool[0, 10] = 124                     # covers 992..999 (the last block, full)
    pool[0, 11] = 5000                    # outside the context: contributes nothing
    pool[1, :3] = [0, 6, 7]               # block 6 = 48..49 only (N = 50); block 7 is beyond
    idx, _ = case.run_reindex(torch.from_numpy(pool).to(DEV), 100)
    idx = idx.cpu().numpy()
    for i in range(2):
        assert np.array_equal(idx[i], case.oracle_reindex(i, pool[i], 100)), i


def test_index_reindex_unsorted_pool_follows_element_order():
    # The header documents an ascending pool (as csa2_index_full writes it); for a row in any
    # other order the selection is the top_k candidates under (score desc, element order asc),
    # written in element order.  Scores from {-1, 0, 1} inputs tie a lot, so the order decides.
    case = IndexCase(W_T + 6, [4000], n_heads=4, qlo=-1, qhi=1)
    blocks = np.random.default_rng(6).permutation(500)[:64].astype(np.int32)   # not ascending
    idx, _ = case.run_reindex(torch.from_numpy(blocks[None].copy()).to(DEV), 100)
    cand = np.concatenate([b * 8 + np.arange(8) for b in blocks])
    s = O.index_scores(case.q[0], case.w[0], case.k[cand])
    chosen = np.sort(np.lexsort((np.arange(cand.size), -s))[:100])           # element positions
    assert np.array_equal(idx.cpu().numpy()[0], cand[chosen])


@pytest.mark.parametrize("pool_blocks,top_k,window", [(2048, 512, 128), (300, 64, 0), (3000, 512, 128), (1, 4, 16),
                                                      (512, 512, 300), (2048, 100, 256), (2048, 700, 128)])
def test_reindex_attend_equals_separate_calls_and_oracle(pool_blocks, top_k, window):
    # csa2_reindex_attend (one call issuing the scoring, selection and attention kernels)
    # against csa2_index_reindex followed by csa2_attend: the same indices and the same attention
    # bit for bit; both against the oracle.  Windows of 300 and 256 give 7 and 3 attention
    # workgroups per query (a cross-workgroup merge); window 0 attends the selection alone.
    lengths = [40000, 777, 0, 16, 25001]
    ic = IndexCase(W_T + 70, lengths, n_heads=4)
    ac = AttendCase(W_T + 70, lengths, n_heads=16, window=max(window, 1), swa_cap=max(window, 128))
    _, pool, _ = ic.run_full(512, pool_blocks)
    q2 = synth.int_bf16(W_T + 70, synth.T_IDX_Q, (len(lengths), 4, 64), seq=5)
    w2 = synth.int_weights(W_T + 70, synth.T_IDX_W, (len(lengths), 4), seq=5)
    q2_dev, w2_dev = bf16_tensor(q2), torch.from_numpy(w2).to(DEV)
    idx_a, _ = ic.run_reindex(pool, top_k, q_dev=q2_dev, w_dev=w2_dev)
    idx_a = idx_a.cpu().numpy()
    scale = 1 / np.sqrt(128)
    n_q = len(lengths)
    out_a = torch.empty((n_q, 16, 128), dtype=torch.float32, device=DEV)
    C.csa2_attend(ac.q_dev, ac.codes, ac.scales, ac.seqs, torch.from_numpy(idx_a).to(DEV), ac.swa_dev,
                  ac.swa_row0_dev, ac.swa_cap, window, scale, out_a)
    ws = C.alloc_workspace(C.csa2_workspace_bytes(C.OP_INDEX_REINDEX, n_q, 0, 0, top_k, pool_blocks))
    idx_b = torch.full((n_q, top_k), -7, dtype=torch.int32, device=DEV)
    out_b = torch.full((n_q, 16, 128), float("nan"), dtype=torch.float32, device=DEV)
    C.csa2_reindex_attend(q2_dev, w2_dev, ic.k_dev, None, ic.seqs, pool, top_k, idx_b, ac.q_dev, ac.codes, ac.scales,
                          ac.swa_dev, ac.swa_row0_dev, ac.swa_cap, window, scale, out_b, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx_b.cpu().numpy(), idx_a)
    assert np.array_equal(out_b.cpu().numpy(), out_a.cpu().numpy())
    pool_np = pool.cpu().numpy()
    for i in range(n_q):
        assert np.array_equal(idx_a[i], ic.oracle_reindex(i, pool_np[i], top_k, q=q2[i], w=w2[i])), i
    ac.window = window
    ac.check(out_b.cpu().numpy(), idx_a, scale)
    ac.check(out_a.cpu().numpy(), idx_a, scale)


# ---------------------------------------------------------------- attention
def test_attend_selected_plus_window():
    lengths = [4096, 300, 130, 5000]
    case = AttendCase(W_T + 5, lengths, n_heads=16, window=128)
    r = np.random.default_rng(11)
    idx = np.full((len(lengths), 512), -1, dtype=np.int64)
    for i, n in enumerate(lengths):
        sel = np.sort(r.choice(n, size=min(n, 400), replace=False))
        idx[i, :sel.size] = sel
    out, _ = case.run(idx, 1 / np.sqrt(128))
    case.check(out, idx, 1 / np.sqrt(128))


@pytest.mark.parametrize("n_heads,top_k,window", [(5, 3, 0), (16, 0, 128), (1, 700, 17), (16, 64, 64)])
def test_attend_shapes(n_heads, top_k, window):
    lengths = [1000, 2, 64]
    case = AttendCase(W_T + 6 + top_k, lengths, n_heads=n_heads, window=window, swa_cap=max(window, 1))
    r = np.random.default_rng(12 + top_k)
    idx = np.full((len(lengths), top_k), -1, dtype=np.int64)
    for i, n in enumerate(lengths):
        m = min(n, top_k)
        idx[i, :m] = r.choice(n, size=m, replace=False)
    out, _ = case.run(idx, 0.125)
    case.check(out, idx, 0.125)


@pytest.mark.parametrize("n_q,top_k,window", [(1, 512, 128), (8, 100, 37), (63, 33, 0), (64, 512, 128),
                                              (65, 512, 128), (5, 0, 100), (4, 0, 512), (3, 1024, 256),
                                              (16, 16, 16)])
def test_attend_decode_split_against_oracle_and_repeatable(n_q, top_k, window):
    # decode-sized calls (<= 64 queries) share each query's entries out over several workgroups
    # and merge their partials through the workspace; 65 queries take one workgroup per query.
    # Lengths include empty, shorter than the window and shorter than top_k; selections hold
    # -1 padding, out-of-range positions and duplicates.  A second call on the same workspace
    # (its counters left zero by the first) gives bit-identical outputs.
    r = np.random.default_rng(1000 + n_q + top_k + window)
    lengths = r.integers(1, 6000, size=n_q)
    lengths[3::7] = 0
    lengths[1::5] = r.integers(1, 40, size=lengths[1::5].size)
    case = AttendCase(W_T + 9, lengths, n_heads=16, window=window, swa_cap=max(window, 1) + 3)
    idx = np.full((n_q, top_k), -1, dtype=np.int64)
    for i, n in enumerate(lengths):
        m = min(int(n), top_k)
        if m:
            idx[i, :m] = r.choice(int(n), size=m, replace=False)
        if top_k >= 4 and n > 0:
            idx[i, top_k - 2] = idx[i, 0]          # a duplicate
            idx[i, top_k - 1] = n + 5              # out of range: skipped
    scale = 1 / np.sqrt(128)
    ws = C.attend_workspace(n_q, top_k, window)
    out1, _ = case.run(idx, scale, ws=ws)
    out2, _ = case.run(idx, scale, ws=ws)
    assert np.array_equal(out1, out2)
    case.check(out1, idx, scale)
    for i, n in enumerate(lengths):
        if n == 0:
            assert np.all(out1[i] == 0.0)


def test_attend_empty_context_is_zero_and_duplicates_count():
    lengths = [0, 10]
    case = AttendCase(W_T + 7, lengths, n_heads=16, window=4)
    idx = np.array([[-1, -1, 3, 3], [3, 3, 9, 12]])         # 12 >= N is ignored; duplicates kept
    out, _ = case.run(idx, 0.1)
    assert np.all(out[0] == 0.0)
    case.check(out, idx, 0.1)


def test_attend_dense_equivalence_all_positions():
    lengths = [512, 200]
    case = AttendCase(W_T + 8, lengths, n_heads=16, window=0, swa_cap=1)
    idx = np.full((2, 512), -1, dtype=np.int64)
    idx[0] = np.arange(512)
    idx[1, :200] = np.arange(200)
    out, _ = case.run(idx, 1 / np.sqrt(128))
    for i, n in enumerate(lengths):
        r0 = int(case.row0[i])
        kv = torch.from_numpy(O.fp4_dequantize(case.codes_ref[r0:r0 + n], case.scales_ref[r0:r0 + n]))
        qt = torch.from_numpy(O.bf16_to_f64(case.q[i]))[None, :, None, :]
        kt = kv[None, None].expand(1, 16, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=1 / np.sqrt(128))[0, :, 0].numpy()
        assert np.abs(out[i] - ref).max() <= 2e-3 * np.abs(kv.numpy()).max()


# ---------------------------------------------------------------- measurement read kernel
@pytest.mark.parametrize("n_words", [4, 1 << 16, (1 << 22) + 12])
def test_stream_read_covers_every_word_once(n_words):
    """The read kernel folds every word it reads with XOR into one word per workgroup: the XOR of
    the sink is the XOR of the whole buffer only if each word is read exactly once."""
    g = np.random.default_rng(n_words)
    x = g.integers(-2**31, 2**31, size=n_words, dtype=np.int64).astype(np.int32)
    sink = torch.full((C.lib().csa2_stream_read_groups(),), 0, dtype=torch.int32, device=DEV)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()
    C.csa2_stream_read(torch.from_numpy(x).to(DEV), sink, ev[0], ev[1])
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy()) == np.bitwise_xor.reduce(x)
    assert ev[0].elapsed_time(ev[1]) >= 0.0
