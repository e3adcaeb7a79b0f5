"""Pins for the oracle's MXFP4 indexer keys ([Article] sections VII and XI: indexer K in
MXFP4, E2M1 elements with one E8M0 scale byte per 32 channels).

References other than the oracle itself: the page's Fmt byte model (golden constants), the
closed form of a block holding one nonzero value, hand-worked blocks, the format's error
bound, and the invariant that integer keys in [-4, 4] are exact, so every score and every
selection equals the bf16-key result.
"""
import json
import os

import numpy as np

import oracle as O
from compressed_sparse_attention_07_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def _bits(vals):
    return synth.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_bytes_per_key_follow_the_page_fmt_model():
    assert GOLD["byte_budget_inputs"]["indexer_format"] == "E2M1 + one E8M0 byte per 32 channels"
    for dim in (64, 128):
        # the page's model: n * bits / 8 + n / scale_block * scale_bytes, with 4 bits, 32, 1 byte
        assert O.mxfp4_entry_bytes(dim) == dim * 4 / 8 + dim / 32 * 1
    assert O.mxfp4_entry_bytes(64) == 34        # vs 128 B for a bf16 key: 3.76x fewer


def test_single_value_block_closed_form_every_bf16():
    # A block whose only nonzero value is x: X = 2^(floor(log2|x|) - 2), so |x| / X lies in
    # [4, 8) and the element is 4 (|x| <= 5X, 5 ties to the even code of 4) or 6.
    bits = np.arange(1, 0x7F80, dtype=np.uint16)              # every positive finite bf16
    f = synth.bf16_bits_to_f32(bits).astype(np.float64)
    e = np.floor(np.log2(f)) - 2
    keep = e >= -126                                           # clamped codes are checked below
    bits, f, e = bits[keep], f[keep], e[keep]
    rows = np.zeros((bits.size, 64), dtype=np.uint16)          # the second block stays all zero
    rows[:, 7] = bits
    rows = np.concatenate([rows, rows | 0x8000])               # and every negative one
    codes, scales = O.mxfp4_quantize(rows)
    X = np.ldexp(1.0, e.astype(np.int64))
    expect = np.where(f <= 5 * X, 4 * X, 6 * X)
    got = O.mxfp4_dequantize(codes, scales)[:, 7]
    assert np.array_equal(got, np.concatenate([expect, -expect]))
    assert np.array_equal(scales[:, 0], np.concatenate([e, e]).astype(np.int64) + 127)
    assert (scales[:, 1] == 1).all()                           # the all-zero second block


def test_hand_worked_blocks():
    rows = np.zeros((5, 32), dtype=np.float32)
    rows[0, 0] = 7.0                  # X = 1, 7 -> saturates to 6
    rows[1, :2] = [1.0, 0.25]         # X = 1/4: 4 and 1, exact
    rows[2, :2] = [3.0, 0.1]          # X = 1/2: 6 and 0.2 -> 0
    rows[3, :3] = [-4.0, 2.5, -1.25]  # X = 1: -4, 2.5 -> 2 (tie to even), -1.25 -> -1 (tie to even)
    codes, scales = O.mxfp4_quantize(_bits(rows))
    dq = O.mxfp4_dequantize(codes, scales)
    assert dq[0, 0] == 6.0 and scales[0, 0] == 127
    assert dq[1, :2].tolist() == [1.0, 0.25] and scales[1, 0] == 125
    assert dq[2, :2].tolist() == [3.0, 0.0] and scales[2, 0] == 126
    assert dq[3, :3].tolist() == [-4.0, 2.0, -1.0]
    assert (dq[4] == 0).all() and scales[4].tolist() == [1]        # all-zero row
    assert codes[0, 0] == 0x07 and codes[3, 0] & 0xF == 0xE          # 6 -> code 7; -4 -> sign | 6


def test_error_bound_on_workload_values():
    x = synth.kv_bf16(5, synth.T_KV, 2000, 64, synth.channel_sigma(5, synth.T_KV_SIGMA, 64))
    codes, scales = O.mxfp4_quantize(x)
    err = np.abs(O.mxfp4_dequantize(codes, scales) - O.bf16_to_f64(x))
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    # nearest rounding: at most half the widest E2M1 gap (2) times X, plus saturation in [6X, 8X)
    assert (err <= 2 * X).all()
    inside = np.abs(O.bf16_to_f64(x)) <= 6 * X
    assert (err[inside] <= X[inside]).all()


def test_integer_keys_are_exact_so_selection_equals_bf16_keys():
    n = 3000
    k = synth.int_bf16(6, synth.T_IDX_K, (n, 64))
    codes, scales = O.mxfp4_quantize(k)
    assert np.array_equal(O.mxfp4_dequantize(codes, scales), O.bf16_to_f64(k))
    q = synth.int_bf16(6, synth.T_IDX_Q, (4, 64))
    w = synth.int_weights(6, synth.T_IDX_W, (4,))
    for top_k, pool in ((512, 64), (16, 3), (4096, 400)):
        a_idx, a_pool = O.index_full(q, w, k, n, top_k, 8, pool)
        b_idx, b_pool = O.index_full_mx(q, w, codes, scales, n, top_k, 8, pool)
        assert np.array_equal(a_idx, b_idx) and np.array_equal(a_pool, b_pool)
        assert np.array_equal(O.index_reindex(q, w, k, n, a_pool, 512, 8),
                              O.index_reindex_mx(q, w, codes, scales, n, a_pool, 512, 8))
