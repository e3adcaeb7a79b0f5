"""Pins for the attention tolerance unit: attended_max_abs and attended_max_abs_fp8 give the
largest |v| over exactly the entries one query attends to, and every attention parity check
scales its bar (2e-3 of that value) by it.

Every expected value below is worked out by hand from the formats' definitions: an E2M1 code
c has magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}[c & 7]; an E4M3 byte with exponent field E (bits
6..3) and mantissa M (bits 2..0) is 2^(E-7) (1 + M/8); a bf16 pattern is the top half of a
binary32.  The cases put a larger value just outside the attended set each time (a position
past the window, a ring row of another query, a row past the visible length, a position before
the replay start, an unselected row), so counting one entry too many changes the result.
"""
import numpy as np

import oracle as O

# bf16 bit patterns
BF_2, BF_3, BF_NEG5, BF_100, BF_1000 = 0x4000, 0x4040, 0xC0A0, 0x42C8, 0x447A
# E4M3 bytes: 1.0, 2.0, 8.0, 16.0 (scales); -8.0, 3.0, 128.0, 448.0 (window values)
E_1, E_2, E_8, E_16 = 0x38, 0x40, 0x50, 0x58
E_NEG8, E_3, E_128, E_448 = 0xD0, 0x44, 0x70, 0x7E


def _fp4_seq(rows=8):
    """An FP4 cache of `rows` positions: position 2 holds +6 x 2 = 12 in channel 0; position 4
    holds -6 x 1 = -6 in channel 11; position 3 holds 6 x 8 = 48 everywhere (never selected);
    position 7 holds 6 x 16 = 96 (outside a length of 6)."""
    codes = np.zeros((rows, 64), np.uint8)
    scales = np.full((rows, 8), E_1, np.uint8)
    codes[2, 0] = 0x07                      # channel 0: code 7 = +6
    scales[2, 0] = E_2                      # group 0 scale 2.0
    codes[4, 5] = 0xF0                      # channel 11: code 0xF = -6 (channel 10: 0)
    codes[3, :] = 0x77
    scales[3, :] = E_8
    codes[7, :] = 0x77
    scales[7, :] = E_16
    return codes, scales


def _bf16_window():
    """A window store of 8 rows: a ring of 4 rows for this query starting at row 4 (position p
    at row 4 + p mod 4), and rows 0-3 belonging to another query's ring (value 1000)."""
    swa = np.zeros((8, 128), np.uint16)
    swa[0:4, :] = BF_1000
    swa[7, 0] = BF_3        # position 3 (and 7, ...)
    swa[4, 10] = BF_NEG5    # position 4 (and 0, ...)
    swa[5, 1] = BF_2        # position 5 (and 1, ...)
    swa[6, 2] = BF_100      # position 6 (and 2, ...)
    return swa


def test_window_only():
    codes, scales = _fp4_seq()
    swa = _bf16_window()
    # n = 6, window 3: positions 3, 4, 5 -> rows 7, 4, 5 -> max(3, 5, 2) = 5 (row 6, position 2,
    # is outside the window and holds 100; rows 0-3 belong to another ring and hold 1000)
    got = O.attended_max_abs(codes, scales, 6, np.full(4, -1), swa, 4, 4, 3)
    assert got == 5.0


def test_selection_with_padding_out_of_range_and_duplicates():
    codes, scales = _fp4_seq()
    swa = _bf16_window()
    # selected {4, 2, 2}: |-6 x 1| = 6 and 6 x 2 = 12; index 7 >= n = 6 is skipped (it would give
    # 96) and so is -1; the window adds 5 -> 12
    got = O.attended_max_abs(codes, scales, 6, np.array([4, -1, 2, 2, 7, -1]), swa, 4, 4, 3)
    assert got == 12.0
    # without position 2 the selection gives 6, the window 5 -> 6
    assert O.attended_max_abs(codes, scales, 6, np.array([4, 4, -1]), swa, 4, 4, 3) == 6.0


def test_window_longer_than_the_context_and_empty_cases():
    codes, scales = _fp4_seq()
    swa = _bf16_window()
    # n = 2, window 3: positions 0 and 1 only (rows 4 and 5) -> max(5, 2) = 5
    assert O.attended_max_abs(codes, scales, 2, np.full(2, -1), swa, 4, 4, 3) == 5.0
    # nothing visible: 0
    assert O.attended_max_abs(codes, scales, 0, np.array([0, 1]), swa, 4, 4, 3) == 0.0
    # window 0 and only an unselected large row present: the selection alone (12)
    assert O.attended_max_abs(codes, scales, 6, np.array([2]), swa, 4, 4, 0) == 12.0


def _e4m3_window():
    """An E4M3 window store, position p at row p (capacity 8)."""
    swa = np.zeros((8, 128), np.uint8)
    swa[2, 0] = E_448
    swa[3, 5] = E_128
    swa[4, 9] = E_NEG8
    swa[5, 127] = E_3
    return swa


def test_fp8_window_replay_bound_drops_the_largest_rows():
    codes, scales = _fp4_seq()
    swa = _e4m3_window()
    # n = 6, window 4 -> positions 2..5; replay start 4 keeps 4 and 5 -> max(8, 3) = 8
    got = O.attended_max_abs_fp8(codes, scales, 6, np.full(4, -1), swa, 0, 8, 4, replay_start=4)
    assert got == 8.0
    # no replay bound: positions 2..5 -> 448; window 3: positions 3..5 -> 128
    assert O.attended_max_abs_fp8(codes, scales, 6, np.full(4, -1), swa, 0, 8, 4) == 448.0
    assert O.attended_max_abs_fp8(codes, scales, 6, np.full(4, -1), swa, 0, 8, 3) == 128.0
    # a replay start past the context: no window at all
    assert O.attended_max_abs_fp8(codes, scales, 6, np.full(4, -1), swa, 0, 8, 4, replay_start=9) == 0.0


def test_fp8_window_with_selection():
    codes, scales = _fp4_seq()
    swa = _e4m3_window()
    # selection {2, 4, 7 (skipped: >= n), -1}: 12; window with replay start 4: 8 -> 12
    got = O.attended_max_abs_fp8(codes, scales, 6, np.array([2, 4, 7, -1]), swa, 0, 8, 4, replay_start=4)
    assert got == 12.0
    # selection {4}: 6 against the window's 8 -> 8
    assert O.attended_max_abs_fp8(codes, scales, 6, np.array([4]), swa, 0, 8, 4, replay_start=4) == 8.0
