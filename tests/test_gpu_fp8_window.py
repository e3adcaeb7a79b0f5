"""GPU parity of the FP8 window store and of attention over it with SWA Bounded Replay
([Article] sections XI and XII), through the C ABI, against the CPU oracle: E4M3 bytes
bit-exact, attention within 2e-3 * max|V| of the oracle's fp64 result."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_attention_07_amd import csa2 as C
from compressed_sparse_attention_07_amd import synth

from gpu_helpers import ATT_TOL, AttendCase, DEV, bf16_tensor

pytestmark = pytest.mark.gpu


def test_fp8_window_append_every_finite_bf16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = synth.bf16_bits_to_f32(bits)
    bits = bits[~np.isnan(f)]                       # inputs are finite or infinite, never NaN
    bits = np.concatenate([bits, np.zeros((-bits.size) % 64, dtype=np.uint16)]).reshape(-1, 64)
    out = torch.full(bits.shape, 0x55, dtype=torch.uint8, device=DEV)
    C.fp8_window_append(bf16_tensor(bits), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), O.e4m3_quantize(bits))


def test_fp8_window_append_scattered_rows():
    x = synth.kv_bf16(21, synth.T_SWA, 40, 128, synth.channel_sigma(21, synth.T_SWA_SIGMA, 128))
    # distinct rows, some outside [0, 40) (skipped); rows 1-4 and 6 are never named
    rows = np.array([5, 0, 39, 7, -1, 100] + [r for r in range(8, 50) if r != 39][:34], dtype=np.int64)
    out = torch.full((40, 128), 0x55, dtype=torch.uint8, device=DEV)
    C.fp8_window_append(bf16_tensor(x), out, dst_rows=torch.from_numpy(rows).to(DEV))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = O.e4m3_quantize(x)
    for t, r in enumerate(rows):
        if 0 <= r < 40:
            assert np.array_equal(got[r], ref[t])
    written = {int(r) for r in rows if 0 <= r < 40}
    for r in range(40):
        if r not in written:
            assert (got[r] == 0x55).all()


class Fp8Case(AttendCase):
    """AttendCase whose window store is converted to E4M3 on the GPU (checked bit-exact)."""

    def __init__(self, *a, **kw):
        super().__init__(*a, **kw)
        self.swa8_ref = O.e4m3_quantize(self.swa)
        self.swa8 = torch.zeros(self.swa.shape, dtype=torch.uint8, device=DEV)
        C.fp8_window_append(self.swa_dev, self.swa8)
        torch.cuda.synchronize()
        assert np.array_equal(self.swa8.cpu().numpy(), self.swa8_ref)

    def run8(self, idx_np, scale, replay=None):
        n_q = len(self.lengths)
        out = torch.full((n_q, self.n_heads, 128), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.from_numpy(np.ascontiguousarray(idx_np.astype(np.int32))).to(DEV)
        rs = None if replay is None else torch.from_numpy(np.asarray(replay, dtype=np.int64)).to(DEV)
        C.csa2_attend_fp8win(self.q_dev, self.codes, self.scales, self.seqs, idx, self.swa8, self.swa_row0_dev,
                             self.swa_cap, self.window, scale, out, replay_start=rs)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def check8(self, out, idx_np, scale, replay=None):
        worst = 0.0
        for i in range(len(self.lengths)):
            r0, n = int(self.row0[i]), int(self.lengths[i])
            s = 0 if replay is None else int(replay[i])
            ref = O.attend_fp8_window(self.q[i], self.codes_ref[r0:r0 + n], self.scales_ref[r0:r0 + n], n,
                                      idx_np[i], self.swa8_ref, int(self.swa_row0[i]), self.swa_cap, self.window,
                                      scale, replay_start=s)
            vmax = O.attended_max_abs_fp8(self.codes_ref[r0:r0 + n], self.scales_ref[r0:r0 + n], n, idx_np[i],
                                          self.swa8_ref, int(self.swa_row0[i]), self.swa_cap, self.window,
                                          replay_start=s)
            err = float(np.abs(out[i].astype(np.float64) - ref).max())
            if vmax == 0.0:
                assert err == 0.0, (i, err)
            else:
                assert err <= ATT_TOL * vmax, (i, err, vmax)
                worst = max(worst, err / vmax)
        return worst


def _idx_for(lengths, top_k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((len(lengths), top_k), -1, dtype=np.int64)
    for i, n in enumerate(lengths):
        k = min(top_k, int(n))
        if k:
            idx[i, :k] = np.sort(rng.choice(int(n), size=k, replace=False))
    return idx


def test_fp8_window_attention_with_replay_starts():
    lengths = [3000, 200, 129, 128, 50, 1, 0, 4096]
    case = Fp8Case(31, lengths, n_heads=16, window=128, swa_cap=128)
    idx = _idx_for(lengths, 512, 31)
    scale = 1 / np.sqrt(128)
    replay = [2950, 0, 100, 127, 60, 0, 0, 5000]    # inside, none, partial, last only, past n, ...
    out = case.run8(idx, scale, replay)
    worst = case.check8(out, idx, scale, replay)
    assert worst < 1e-3
    out0 = case.run8(idx, scale, None)              # no bound: the plain window
    case.check8(out0, idx, scale, None)


def test_fp8_window_only_and_short_selection():
    lengths = [1000, 700, 64]
    case = Fp8Case(32, lengths, n_heads=8, window=128, swa_cap=256)
    idx = np.full((3, 16), -1, dtype=np.int64)       # nothing selected: the window alone
    scale = 0.125
    case.check8(case.run8(idx, scale, [0, 650, 0]), idx, scale, [0, 650, 0])
    idx2 = _idx_for(lengths, 16, 32)                 # a 16-entry selection (one FP4 block)
    case.check8(case.run8(idx2, scale, [990, 0, 63]), idx2, scale, [990, 0, 63])


def test_fp8_window_many_queries_several_rounds():
    # top_k 1024 and window 256: two rounds per wave
    lengths = list(synth.log_uniform_lengths(33, 40, 300, 5000))
    case = Fp8Case(33, lengths, n_heads=16, window=256, swa_cap=256)
    idx = _idx_for(lengths, 1024, 33)
    rng = np.random.default_rng(33)
    replay = [int(rng.integers(0, n + 1)) for n in lengths]
    scale = 1 / np.sqrt(128)
    case.check8(case.run8(idx, scale, replay), idx, scale, replay)


@pytest.mark.parametrize("window,cap,top_k", [(128, 128, 512), (256, 300, 1024), (16, 16, 16)])
def test_new_window_vector_attended_and_written(window, cap, top_k):
    # win_new: the step's own window vector per query ([Article] section VI: every layer computes
    # its own window entries).  The call attends it as position N - 1 and writes it to that row of
    # the store (E4M3 for an FP8 store), also when a replay start keeps it out of the window; the
    # store's old row is never read (it holds a marker here).
    lengths = [3000, 129, 1, 700, 0, 4096]
    n_q = len(lengths)
    for fp8 in (False, True):
        case = Fp8Case(34, lengths, n_heads=16, window=window, swa_cap=cap)
        new = synth.kv_bf16(34, synth.T_SWA_NEW, n_q, 128, synth.channel_sigma(34, synth.T_SWA_SIGMA, 128))
        rows = np.array([i * cap + (n - 1) % cap for i, n in enumerate(lengths) if n > 0])
        truth = case.swa.copy()
        truth[rows] = new[[i for i, n in enumerate(lengths) if n > 0]]
        before = truth.copy()
        before[rows] = 0x447A                                   # bf16 1000: a marker the call overwrites
        idx = _idx_for(lengths, top_k, 34)
        scale = 1 / np.sqrt(128)
        replay = [2990, 0, 0, 700, 0, 0]                       # query 3's window excludes position N - 1
        out = torch.full((n_q, 16, 128), float("nan"), dtype=torch.float32, device=DEV)
        idx_t = torch.from_numpy(idx.astype(np.int32)).to(DEV)
        if fp8:
            store = torch.zeros(before.shape, dtype=torch.uint8, device=DEV)
            C.fp8_window_append(bf16_tensor(before), store)
            C.csa2_attend_fp8win(case.q_dev, case.codes, case.scales, case.seqs, idx_t, store, case.swa_row0_dev,
                                 cap, window, scale, out, replay_start=torch.tensor(replay, device=DEV),
                                 win_new=bf16_tensor(new))
        else:
            store = bf16_tensor(before)
            C.csa2_attend(case.q_dev, case.codes, case.scales, case.seqs, idx_t, store, case.swa_row0_dev, cap,
                          window, scale, out, win_new=bf16_tensor(new))
        torch.cuda.synchronize()
        got_store = store.cpu().numpy() if fp8 else store.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got_store, O.e4m3_quantize(truth) if fp8 else truth), fp8
        res = out.cpu().numpy()
        for i, n in enumerate(lengths):
            r0 = int(case.row0[i])
            if fp8:
                s8 = O.e4m3_quantize(truth)
                ref = O.attend_fp8_window(case.q[i], case.codes_ref[r0:r0 + n], case.scales_ref[r0:r0 + n], n,
                                          idx[i], s8, i * cap, cap, window, scale, replay_start=replay[i])
                vmax = O.attended_max_abs_fp8(case.codes_ref[r0:r0 + n], case.scales_ref[r0:r0 + n], n, idx[i],
                                              s8, i * cap, cap, window, replay_start=replay[i])
            else:
                ref = O.attend(case.q[i], case.codes_ref[r0:r0 + n], case.scales_ref[r0:r0 + n], n, idx[i], truth,
                               i * cap, cap, window, scale)
                vmax = O.attended_max_abs(case.codes_ref[r0:r0 + n], case.scales_ref[r0:r0 + n], n, idx[i], truth,
                                          i * cap, cap, window)
            err = float(np.abs(res[i].astype(np.float64) - ref).max())
            assert err <= ATT_TOL * vmax if vmax > 0 else err == 0.0, (fp8, i, err, vmax)
