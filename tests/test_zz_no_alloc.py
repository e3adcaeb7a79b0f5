"""The no-allocation Reindex entry point against the workspace one, through the C ABI: two
calls in a row on one GPU (the second with fewer queries and a smaller pool), bit-identical
indices; then the size limits."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_07_amd import csa2 as C
from compressed_sparse_attention_07_amd import synth

from gpu_helpers import DEV, IndexCase, bf16_tensor

pytestmark = pytest.mark.gpu


def _pair(case, pool, top_k, q2, w2):
    n_q = len(case.lengths)
    ws = C.alloc_workspace(C.csa2_workspace_bytes(C.OP_INDEX_REINDEX, n_q, 0, 0, top_k, pool.shape[1]))
    a = torch.full((n_q, top_k), -7, dtype=torch.int32, device=DEV)
    C.csa2_index_reindex(q2, w2, case.k_dev, case.seqs, pool, top_k, a, ws)
    b = torch.full((n_q, top_k), -9, dtype=torch.int32, device=DEV)
    C.csa2_index_reindex_noalloc(q2, w2, case.k_dev, case.seqs, pool, top_k, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_reindex_equals_workspace_call_twice():
    # first call: 64 queries (the limit), 2,048-block pools; second: 5 queries, 300-block pools
    for lengths, pool_blocks, top_k, seed in (
            (list(synth.log_uniform_lengths(61, 64, 2000, 200000)), 2048, 512, 1),
            ([40000, 777, 0, 16, 25001], 300, 64, 2)):
        case = IndexCase(961 + seed, lengths, n_heads=4)
        _, pool, _ = case.run_full(512, pool_blocks)
        q2 = synth.int_bf16(961 + seed, synth.T_IDX_Q, (len(lengths), 4, 64), seq=5)
        w2 = synth.int_weights(961 + seed, synth.T_IDX_W, (len(lengths), 4), seq=5)
        a, b = _pair(case, pool, top_k, bf16_tensor(q2), torch.from_numpy(w2).to(DEV))
        assert np.array_equal(a, b), (len(lengths), pool_blocks)
        pool_np = pool.cpu().numpy()
        for i in range(len(lengths)):   # and against the oracle
            assert np.array_equal(b[i], case.oracle_reindex(i, pool_np[i], top_k, q=q2[i], w=w2[i])), i


def test_noalloc_reindex_rejects_sizes_past_its_scratch():
    case = IndexCase(970, [1000] * 65, n_heads=4)
    pool = torch.zeros((65, 16), dtype=torch.int32, device=DEV)
    out = torch.zeros((65, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(C.Csa2Error) as e:
        C.csa2_index_reindex_noalloc(case.q_dev, case.w_dev, case.k_dev, case.seqs, pool, 8, out)
    assert e.value.status == C.ERR_SCRATCH
    case2 = IndexCase(971, [1000], n_heads=4)
    pool2 = torch.zeros((1, 2049), dtype=torch.int32, device=DEV)
    with pytest.raises(C.Csa2Error) as e:
        C.csa2_index_reindex_noalloc(case2.q_dev, case2.w_dev, case2.k_dev, case2.seqs, pool2, 8, out[:1])
    assert e.value.status == C.ERR_SCRATCH
