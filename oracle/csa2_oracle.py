"""Plain fp64 CPU oracle for CSA2 compressed sparse attention over an FP4 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may import,
call or execute this module; only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

Sources (the three web pages the method is described on):
  [Viz]     visualisation page "DeepSeek-V4.1-Flash: shrinking KV cache at 552B
            scale" (podcast.do-not-panic.com), figure captions.
  [Summary] "DeepSeek Cuts KV Cache Footprint Fourfold" (sotapapers.com),
            section "Technical Approach".
  [Article] "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per
            Token" (trishampatil.com), sections VI, VII, VIII, IX, XI, XII.

Conventions: bf16 tensors arrive as uint16 bit patterns and are widened exactly
to fp64.  Every computation is fp64 with plain loops or a single library
primitive (matmul, sort) per step, in the order the pages describe.

Readings where the pages are silent (each is listed, with its reason, in the
design notes of this repository):
  * the indexer score of position p is sum_h w_h * max(0, q_h . k_p) -- the
    pages name a "lightning-style" indexer without printing its formula, so
    this function is PARITY UNPINNED with respect to the pages (it is pinned
    only by brute force and closed forms);
  * FP4 rounding is round-to-nearest, ties-to-even, for both the E4M3 scale
    (of amax/6) and the E2M1 elements (of x/scale), saturating at 6;
  * the sign bit of an element's code is the sign bit of its bf16 input;
  * low nibble = even channel; one scale byte per 16 channels;
  * ties in every ranking go to the lower position (or block) index;
  * selection outputs are in ascending index order, padded with -1;
  * attention is one softmax over the selected entries followed by the window
    entries (no de-duplication), with keys equal to values;
  * an FP8 window stores each value as the nearest E4M3 ('fn') value, ties to even,
    saturating at +-448 (the format has no infinity), with the value's sign bit and no
    scale; a replay start s limits a query's window to positions >= s;
  * MXFP4 indexer keys (E2M1 + one E8M0 byte per 32 channels) follow the microscaling
    conversion: the block's scale is 2^(floor(log2 amax) - 2) (2 = the exponent of E2M1's
    largest value 6), its code clamped to [1, 254] (so an all-zero or vanishing block uses
    2^-126), each element the E2M1 value nearest to x / scale (ties to even, beyond 6 -> 6)
    with x's sign bit.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Formats  ([Viz] FP4 caption; [Article] section XI: E2M1 elements with one
# E4M3 scale per 16 channels, no second-level global scale)
# ---------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m                       # subnormal: m * 2^(1-1) * 1/2
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return sign * mag


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 ('fn') byte: sign bit 7, exponent bits 6..3 (bias 7), mantissa 2..0.
    There are no infinities; S.1111.111 is NaN, so the largest finite magnitude is 448."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    E = (code >> 3) & 15
    M = code & 7
    if E == 15 and M == 7:
        return float("nan")
    if E == 0:
        return sign * 2.0 ** -6 * (M / 8.0)
    return sign * 2.0 ** (E - 7) * (1.0 + M / 8.0)


E2M1_MAGNITUDES = np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)   # codes 0..7
E4M3_NONNEG = np.array([e4m3_value(c) for c in range(127)], dtype=np.float64)       # codes 0..126 (finite, >= 0)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _nearest_even(dist: np.ndarray) -> np.ndarray:
    """Index of the smallest entry along the last axis; among equal smallest entries,
    the even index (round half to even: two tied candidates are always adjacent codes)."""
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    idx = np.arange(dist.shape[-1])
    # prefer an even index among the tied ones, else the (unique) odd one
    even_pick = np.where(tied & (idx % 2 == 0), idx, dist.shape[-1] + 1).min(axis=-1)
    any_pick = np.where(tied, idx, dist.shape[-1] + 1).min(axis=-1)
    return np.where(even_pick <= dist.shape[-1], even_pick, any_pick)


def fp4_quantize(x_bf16: np.ndarray, group: int = 16):
    """Quantise post-RoPE vectors to FP4 ([Article] section XI, [Viz] FP4 caption).

    x_bf16: uint16 [T, D] bf16 bits, D % 16 == 0.
    Returns codes uint8 [T, D/2] (channel 2i in the low nibble of byte i, 2i+1 in the
    high nibble) and scales uint8 [T, D/16] (E4M3 byte of channels [16j, 16j+16)).

    Per 16-channel group: amax = max |x|; the scale s is the E4M3 value nearest to
    amax/6 (6 = largest E2M1 magnitude), ties to even; each element's code is the
    E2M1 value nearest to x/s (ties to even, beyond 6 -> 6), with x's sign bit.
    If s == 0 every magnitude code is 0.  Distances are computed as |6*v - amax| and
    |m*s - |x|| which are exact in fp64 for bf16 inputs and these formats.
    """
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    T, D = x_bf16.shape
    assert D % group == 0
    packed = np.empty((T, D // 2), dtype=np.uint8)
    scale_code = np.empty((T, D // group), dtype=np.uint8)
    for r0 in range(0, T, 4096):                 # row chunks only bound host memory
        r1 = min(T, r0 + 4096)
        packed[r0:r1], scale_code[r0:r1] = _fp4_quantize_rows(x_bf16[r0:r1], group)
    return packed, scale_code


def _fp4_quantize_rows(x_bf16: np.ndarray, group: int):
    T, D = x_bf16.shape
    x = bf16_to_f64(x_bf16).reshape(T, D // group, group)
    sign = ((x_bf16 >> 15) & 1).astype(np.uint8).reshape(T, D // group, group)
    amax = np.abs(x).max(axis=-1)                                            # [T, G]
    # nearest E4M3 to amax/6  <=>  smallest |6 v - amax|
    dist_s = np.abs(6.0 * E4M3_NONNEG[None, None, :] - amax[..., None])      # [T, G, 127]
    scale_code = _nearest_even(dist_s).astype(np.uint8)                      # [T, G]
    s = E4M3_NONNEG[scale_code]                                              # [T, G]
    # nearest E2M1 magnitude to |x|/s  <=>  smallest |m s - |x||  (s > 0)
    dist_e = np.abs(E2M1_MAGNITUDES[None, None, None, :] * s[..., None, None] - np.abs(x)[..., None])
    mag = _nearest_even(dist_e).astype(np.uint8)                             # [T, G, 16]
    mag = np.where(s[..., None] == 0.0, np.uint8(0), mag)
    code = (sign << 3) | mag
    code = code.reshape(T, D)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_code


def fp4_dequantize(codes: np.ndarray, scales: np.ndarray, group: int = 16) -> np.ndarray:
    """fp64 values v = E2M1(code) * E4M3(scale) ([Article] section XI: values are
    dequantised before attention).  codes uint8 [T, D/2], scales uint8 [T, D/16]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    T = codes.shape[0]
    D = codes.shape[1] * 2
    c = np.empty((T, D), dtype=np.uint8)
    c[:, 0::2] = codes & 0xF
    c[:, 1::2] = codes >> 4
    table = np.array([e2m1_value(k) for k in range(16)], dtype=np.float64)
    s = np.array([e4m3_value(k) for k in range(256)], dtype=np.float64)[scales]   # [T, G]
    return table[c] * np.repeat(s, group, axis=1)


def fp4_entry_bytes(dim: int, group: int = 16) -> int:
    """Bytes per cached FP4 entry: 4 bits per value plus one scale byte per group."""
    return dim // 2 + dim // group


# ---------------------------------------------------------------------------
# Indexer ([Article] section IX; [Summary] Technical Approach)
# ---------------------------------------------------------------------------


def index_scores(q_bf16: np.ndarray, w: np.ndarray, k_bf16: np.ndarray) -> np.ndarray:
    """Score every key row: s_p = sum_h w_h * max(0, q_h . k_p).

    q_bf16 [Hi, Di] bf16 bits, w [Hi] fp32, k_bf16 [N, Di] bf16 bits -> fp64 [N].
    PARITY UNPINNED with respect to the pages: they do not print the formula.
    """
    q = bf16_to_f64(q_bf16)
    k = bf16_to_f64(k_bf16)
    dots = k @ q.T                                   # [N, Hi]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def select_top(values: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """The first min(k, len) ids under the order (value descending, id ascending),
    returned in ascending id order and padded with -1 to length k."""
    values = np.asarray(values, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -values))               # primary: -value, secondary: id
    chosen = np.sort(ids[order[:k]])
    out = np.full(k, -1, dtype=np.int64)
    out[: chosen.size] = chosen
    return out


def block_max(scores: np.ndarray, block: int) -> np.ndarray:
    """Block score = max index score over the block's valid positions ([Article] section IX,
    Figure 4 caption).  Blocks are [block*b, block*b + block) clipped to the context."""
    n = scores.shape[0]
    nb = -(-n // block)
    return np.array([scores[b * block: min(n, b * block + block)].max() for b in range(nb)],
                    dtype=np.float64)


def index_full(q_bf16, w, k_bf16_seq, n: int, top_k: int, block: int = 8, pool_blocks: int = 0):
    """Full mode for one query: score all n visible positions, take Top-K over the whole
    context and, if pool_blocks > 0, the top pool_blocks blocks by block-max score
    ([Article] section IX; [Summary] Technical Approach).

    k_bf16_seq: the sequence's indexer keys, row p = position p (at least n rows).
    Returns (idx int64 [top_k], pool int64 [pool_blocks] or None)."""
    s = index_scores(q_bf16, w, k_bf16_seq[:n])
    idx = select_top(s, np.arange(n), top_k)
    pool = None
    if pool_blocks > 0:
        bm = block_max(s, block) if n > 0 else np.zeros(0)
        pool = select_top(bm, np.arange(bm.shape[0]), pool_blocks)
    return idx, pool


def index_reindex(q_bf16, w, k_bf16_seq, n: int, pool: np.ndarray, top_k: int, block: int = 8):
    """Reindex mode for one query: Top-K among the positions of the pool's blocks,
    scored with this layer's own query against the Full layer's keys
    ([Article] sections VIII-IX; [Summary] Technical Approach)."""
    blocks = np.asarray(pool, dtype=np.int64)
    blocks = blocks[blocks >= 0]
    cand = np.array(sorted(p for b in blocks for p in range(b * block, b * block + block) if p < n),
                    dtype=np.int64)
    s = index_scores(q_bf16, w, k_bf16_seq[cand]) if cand.size else np.zeros(0)
    return select_top(s, cand, top_k)


# ---------------------------------------------------------------------------
# MXFP4 indexer keys ([Article] sections VII and XI: indexer K in MXFP4, E2M1 elements with
# one E8M0 scale byte per 32 channels)
# ---------------------------------------------------------------------------


def mxfp4_quantize(x_bf16: np.ndarray, block: int = 32):
    """bf16 bits [T, D] (D % 32 == 0) -> (codes uint8 [T, D/2], scales uint8 [T, D/32]).

    Scale of a 32-channel block: X = 2^e with e = floor(log2 amax) - 2, its E8M0 code e + 127
    clamped to [1, 254] (an all-zero block gets code 1).  Element: the E2M1 magnitude nearest
    to |x| / X (ties to the even code, beyond 6 -> 6) with x's sign bit.  Distances
    |m X - |x|| are exact in fp64 (X is a power of two, m has two significant bits).
    Byte i of a row holds channel 2i in its low nibble and 2i + 1 in its high nibble."""
    x_bf16 = np.asarray(x_bf16, dtype=np.uint16)
    T, D = x_bf16.shape
    assert D % block == 0
    if T > 4096:                                   # row chunks only bound host memory
        parts = [mxfp4_quantize(x_bf16[r0:r0 + 4096], block) for r0 in range(0, T, 4096)]
        return np.concatenate([a for a, _ in parts]), np.concatenate([b for _, b in parts])
    x = bf16_to_f64(x_bf16).reshape(T, D // block, block)
    sign = ((x_bf16 >> 15) & 1).astype(np.uint8).reshape(T, D // block, block)
    amax = np.abs(x).max(axis=-1)                                  # [T, G]
    _, ex = np.frexp(amax)                                         # amax = m 2^ex, m in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - 2, -127)                       # floor(log2 amax) - 2
    code = np.clip(e + 127, 1, 254).astype(np.uint8)
    X = np.ldexp(1.0, code.astype(np.int64) - 127)                 # [T, G]
    dist = np.abs(E2M1_MAGNITUDES[None, None, None, :] * X[..., None, None] - np.abs(x)[..., None])
    mag = _nearest_even(dist).astype(np.uint8)
    c = ((sign << 3) | mag).reshape(T, D)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return packed, code


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """fp64 values E2M1(code) * 2^(scale - 127)."""
    codes = np.asarray(codes, dtype=np.uint8)
    T, D = codes.shape[0], codes.shape[1] * 2
    c = np.empty((T, D), dtype=np.uint8)
    c[:, 0::2] = codes & 0xF
    c[:, 1::2] = codes >> 4
    table = np.array([e2m1_value(k) for k in range(16)], dtype=np.float64)
    X = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return table[c] * np.repeat(X, block, axis=1)


def mxfp4_entry_bytes(dim: int, block: int = 32) -> int:
    """Bytes per MXFP4 key: 4 bits per value plus one E8M0 byte per block."""
    return dim // 2 + dim // block


def index_scores_f64(q_bf16: np.ndarray, w: np.ndarray, k: np.ndarray) -> np.ndarray:
    """index_scores with the keys given as fp64 values (e.g. dequantised MXFP4 keys)."""
    q = bf16_to_f64(q_bf16)
    dots = np.asarray(k, dtype=np.float64) @ q.T
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def index_full_mx(q_bf16, w, k_codes_seq, k_scales_seq, n: int, top_k: int, block: int = 8,
                  pool_blocks: int = 0):
    """index_full over MXFP4 keys: the same scores and selection on the dequantised keys."""
    s = index_scores_f64(q_bf16, w, mxfp4_dequantize(k_codes_seq[:n], k_scales_seq[:n])) if n > 0 \
        else np.zeros(0)
    idx = select_top(s, np.arange(n), top_k)
    pool = None
    if pool_blocks > 0:
        bm = block_max(s, block) if n > 0 else np.zeros(0)
        pool = select_top(bm, np.arange(bm.shape[0]), pool_blocks)
    return idx, pool


def index_reindex_mx(q_bf16, w, k_codes_seq, k_scales_seq, n: int, pool: np.ndarray, top_k: int,
                     block: int = 8):
    """index_reindex over MXFP4 keys."""
    blocks = np.asarray(pool, dtype=np.int64)
    blocks = blocks[blocks >= 0]
    cand = np.array(sorted(p for b in blocks for p in range(b * block, b * block + block) if p < n),
                    dtype=np.int64)
    s = index_scores_f64(q_bf16, w, mxfp4_dequantize(k_codes_seq[cand], k_scales_seq[cand])) \
        if cand.size else np.zeros(0)
    return select_top(s, cand, top_k)


# ---------------------------------------------------------------------------
# Attention ([Article] section VI "What one layer looks like", section XI)
# ---------------------------------------------------------------------------


def e4m3_quantize(x_bf16: np.ndarray) -> np.ndarray:
    """bf16 bits (any shape) -> E4M3 ('fn') bytes ([Article] section XI: the recent-window cache
    stays at FP8).  Each value becomes the nearest finite E4M3 value (distances |v - |x|| are
    exact in fp64), ties to the even code; magnitudes beyond 448 saturate to 448; bit 7 is
    the input's sign bit (so -0 -> 0x80)."""
    xb = np.asarray(x_bf16, dtype=np.uint16)
    # saturate first: past 448 the distances below would no longer be exact in fp64
    mag = np.minimum(np.abs(bf16_to_f64(xb)), 448.0).ravel()
    out = np.empty(mag.shape, dtype=np.uint8)
    for c0 in range(0, mag.size, 1 << 15):       # chunks only bound host memory
        a = mag[c0:c0 + (1 << 15)]
        out[c0:c0 + a.size] = _nearest_even(np.abs(E4M3_NONNEG[None, :] - a[:, None]))
    sign = ((xb >> 15) & 1).astype(np.uint8).ravel()
    return (out | (sign << 7)).reshape(xb.shape)


def e4m3_dequantize(codes: np.ndarray) -> np.ndarray:
    """fp64 values of E4M3 ('fn') bytes."""
    table = np.array([e4m3_value(k) for k in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def _attend_rows(q: np.ndarray, kv: np.ndarray, softmax_scale: float) -> np.ndarray:
    """Softmax attention of the [H, D] query over the rows of kv (keys = values), fp64."""
    logits = (q @ kv.T) * softmax_scale              # [H, E]
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ kv


def attend(q_bf16: np.ndarray, codes_seq: np.ndarray, scales_seq: np.ndarray, n: int,
           idx: np.ndarray, swa_bf16: np.ndarray, swa_row0: int, swa_cap: int,
           window: int, softmax_scale: float) -> np.ndarray:
    """One query's output over its selected FP4 entries plus its recent window.

    q_bf16 [H, D]; codes_seq/scales_seq: the sequence's FP4 cache, row p = position p;
    idx: selected positions (entries outside [0, n) are ignored, so -1 padding drops out);
    swa_bf16: window store, position p at row swa_row0 + (p mod swa_cap);
    the window is positions [max(0, n - window), n).
    Keys and values are the same latent vector.  One softmax runs over the selected
    entries followed by the window entries.  Returns fp64 [H, D] (zeros if nothing is visible).
    """
    q = bf16_to_f64(q_bf16)
    sel = [int(j) for j in np.asarray(idx).ravel() if 0 <= int(j) < n]
    win = list(range(max(0, n - window), n))
    rows = []
    if sel:
        rows.append(fp4_dequantize(codes_seq[sel], scales_seq[sel]))
    if win:
        wrows = [swa_row0 + (p % swa_cap) for p in win]
        rows.append(bf16_to_f64(swa_bf16[wrows]))
    if not rows:
        return np.zeros_like(q)
    kv = np.concatenate(rows, axis=0)                # [E, D]
    return _attend_rows(q, kv, softmax_scale)


def window_positions(n: int, window: int, replay_start: int = 0) -> list:
    """Window of the query that sees [0, n): positions [max(replay_start, n - window), n)
    ([Article] section XII, SWA Bounded Replay: a query at position i attends window keys
    in [max(s, i - win + 1), i]; the decode query is position i = n - 1)."""
    return list(range(max(0, replay_start, n - window), n))


def attend_fp8_window(q_bf16: np.ndarray, codes_seq: np.ndarray, scales_seq: np.ndarray, n: int,
                      idx: np.ndarray, swa_e4m3: np.ndarray, swa_row0: int, swa_cap: int,
                      window: int, softmax_scale: float, replay_start: int = 0) -> np.ndarray:
    """As attend(), with the window read from an E4M3 store ([Article] section XI) and limited
    by a replay start ([Article] section XII): the window is window_positions(n, window,
    replay_start); position p at row swa_row0 + (p mod swa_cap)."""
    q = bf16_to_f64(q_bf16)
    sel = [int(j) for j in np.asarray(idx).ravel() if 0 <= int(j) < n]
    win = window_positions(n, window, replay_start)
    rows = []
    if sel:
        rows.append(fp4_dequantize(codes_seq[sel], scales_seq[sel]))
    if win:
        rows.append(e4m3_dequantize(swa_e4m3[[swa_row0 + (p % swa_cap) for p in win]]))
    if not rows:
        return np.zeros_like(q)
    return _attend_rows(q, np.concatenate(rows, axis=0), softmax_scale)


def attended_max_abs_fp8(codes_seq, scales_seq, n, idx, swa_e4m3, swa_row0, swa_cap, window,
                         replay_start=0) -> float:
    """max |v| over the entries attend_fp8_window attends to."""
    sel = [int(j) for j in np.asarray(idx).ravel() if 0 <= int(j) < n]
    m = 0.0
    if sel:
        m = max(m, float(np.abs(fp4_dequantize(codes_seq[sel], scales_seq[sel])).max()))
    win = window_positions(n, window, replay_start)
    if win:
        m = max(m, float(np.abs(e4m3_dequantize(swa_e4m3[[swa_row0 + (p % swa_cap) for p in win]])).max()))
    return m


def attended_max_abs(codes_seq, scales_seq, n, idx, swa_bf16, swa_row0, swa_cap, window) -> float:
    """max |v| over the entries one query attends to (the tolerance unit for attention parity)."""
    sel = [int(j) for j in np.asarray(idx).ravel() if 0 <= int(j) < n]
    m = 0.0
    if sel:
        m = max(m, float(np.abs(fp4_dequantize(codes_seq[sel], scales_seq[sel])).max()))
    win = list(range(max(0, n - window), n))
    if win:
        m = max(m, float(np.abs(bf16_to_f64(swa_bf16[[swa_row0 + (p % swa_cap) for p in win]])).max()))
    return m
