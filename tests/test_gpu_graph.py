"""A decode step captured in a HIP graph gives, on every replay, exactly what the eager step
gives, with eager work and synchronisations between replays (graph replays must not depend on
state a memset node would have to restore)."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_07_amd import workloads as W

pytestmark = pytest.mark.gpu


def _outputs(r):
    outs = [L.out.clone() for L in r.layers]
    idx = [L.idx.clone() for L in r.layers if L.idx is not None]
    pool = [r.pool.clone()] if r.pool is not None else []
    return outs + idx + pool


def test_graph_replays_match_eager_step():
    wl = W.Workload(60, "graph_b4_20k_6layers", 4, 20000, "FRUURU", 512)
    r = W.Runner(wl, copies=2)
    r.step(copy=0)
    torch.cuda.synchronize()
    ref = _outputs(r)
    graphs = r.capture()
    for rep in range(4):
        for L in r.layers:
            L.out.fill_(float("nan"))
            if L.idx is not None:
                L.idx.fill_(-9)
        r.step(copy=1)                     # eager work between replays
        torch.cuda.synchronize()
        graphs[rep % 2].replay()
        torch.cuda.synchronize()
        got = _outputs(r)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep}"
