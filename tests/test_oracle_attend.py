"""Pins for the oracle's gather-dequant attention.

References other than the oracle itself: torch's scaled_dot_product_attention in fp64
on the CPU (dense special cases), the uniform-softmax closed form (q = 0 gives the
plain mean of every attended entry, duplicates included), and single-entry cases.
"""
import numpy as np
import torch

import oracle as O
from compressed_sparse_attention_07_amd import synth


def _cache(seed, n, d=128):
    sig = synth.channel_sigma(seed, synth.T_KV_SIGMA, d)
    x = synth.kv_bf16(seed, synth.T_KV, n, d, sig)
    codes, scales = O.fp4_quantize(x)
    return codes, scales


def _window(seed, cap, d=128):
    sig = synth.channel_sigma(seed, synth.T_SWA_SIGMA, d)
    return synth.kv_bf16(seed, synth.T_SWA, cap, d, sig)


def _sdpa(q, kv, scale):
    qt = torch.from_numpy(q)[None, :, None, :]                    # [1, H, 1, D]
    kt = torch.from_numpy(kv)[None, None].expand(1, q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    return out[0, :, 0, :].numpy()


def test_all_positions_no_window_is_dense_attention():
    n, h = 300, 16
    codes, scales = _cache(1, n)
    q = synth.normal_bf16(1, synth.T_Q, (h, 128))
    idx = np.arange(n)
    swa = _window(1, 128)
    got = O.attend(q, codes, scales, n, idx, swa, 0, 128, 0, 1 / np.sqrt(128))
    ref = _sdpa(O.bf16_to_f64(q), O.fp4_dequantize(codes, scales), 1 / np.sqrt(128))
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_window_only_is_dense_window_attention():
    n, cap, h = 1000, 128, 16
    codes, scales = _cache(2, n)
    swa = _window(2, cap)
    q = synth.normal_bf16(2, synth.T_Q, (h, 128))
    idx = np.full(512, -1)
    got = O.attend(q, codes, scales, n, idx, swa, 0, cap, 128, 1 / np.sqrt(128))
    rows = [p % cap for p in range(n - 128, n)]
    ref = _sdpa(O.bf16_to_f64(q), O.bf16_to_f64(swa[rows]), 1 / np.sqrt(128))
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_joint_softmax_over_selection_then_window():
    n, cap, h = 500, 128, 4
    codes, scales = _cache(3, n)
    swa = _window(3, cap)
    q = synth.normal_bf16(3, synth.T_Q, (h, 128))
    idx = np.array([5, 77, 499, 130, -1, -1])
    got = O.attend(q, codes, scales, n, idx, swa, 0, cap, 50, 0.3)
    kv = np.concatenate([O.fp4_dequantize(codes[[5, 77, 499, 130]], scales[[5, 77, 499, 130]]),
                         O.bf16_to_f64(swa[[p % cap for p in range(450, 500)]])])
    assert np.allclose(got, _sdpa(O.bf16_to_f64(q), kv, 0.3), rtol=0, atol=1e-12)


def test_zero_query_gives_mean_of_all_attended_entries_with_duplicates():
    n, cap = 64, 128
    codes, scales = _cache(4, n)
    swa = _window(4, cap)
    q = np.zeros((2, 128), dtype=np.uint16)
    idx = np.array([60, 61, 62, 63])                  # also inside the window: counted twice
    got = O.attend(q, codes, scales, n, idx, swa, 0, cap, 8, 1.0)
    sel = O.fp4_dequantize(codes[60:64], scales[60:64])
    win = O.bf16_to_f64(swa[56:64])
    mean = (sel.sum(0) + win.sum(0)) / 12.0
    assert np.allclose(got, mean[None], rtol=0, atol=1e-13)


def test_single_entry_returns_its_value():
    n = 40
    codes, scales = _cache(5, n)
    q = synth.normal_bf16(5, synth.T_Q, (16, 128))
    got = O.attend(q, codes, scales, n, np.array([17, -1, -1]), np.zeros((1, 128), np.uint16), 0, 1, 0, 0.1)
    v = O.fp4_dequantize(codes[17:18], scales[17:18])
    assert np.array_equal(got, np.repeat(v, 16, axis=0))


def test_window_ring_addressing_and_out_of_range_indices():
    n, cap = 1000, 128
    codes, scales = _cache(6, n)
    swa = _window(6, 3 * cap)
    q = synth.normal_bf16(6, synth.T_Q, (16, 128))
    # ring of capacity 128 starting at row 128 of the store; ids >= n are ignored
    got = O.attend(q, codes, scales, n, np.array([3, n, n + 5, -1]), swa, cap, cap, 16, 0.2)
    kv = np.concatenate([O.fp4_dequantize(codes[[3]], scales[[3]]),
                         O.bf16_to_f64(swa[[cap + (p % cap) for p in range(n - 16, n)]])])
    assert np.allclose(got, _sdpa(O.bf16_to_f64(q), kv, 0.2), rtol=0, atol=1e-12)


def test_empty_context_gives_zeros():
    q = synth.normal_bf16(7, synth.T_Q, (16, 128))
    got = O.attend(q, np.zeros((1, 64), np.uint8), np.zeros((1, 8), np.uint8), 0,
                   np.full(8, -1), np.zeros((1, 128), np.uint16), 0, 1, 128, 0.1)
    assert np.array_equal(got, np.zeros((16, 128)))
