"""Seeded synthetic inputs for the CSA2 hot path.

This module only draws random numbers and stores them in the storage types the
path consumes (bf16 bit patterns as uint16, fp32 weights, int64 row offsets).
It holds none of the method's arithmetic: no quantisation, scoring, selection
or attention.  Both the HIP path and the CPU oracle are fed from here.

Every stream is numpy PCG64 seeded with SeedSequence([0xC5A2, workload, tensor, seq]) (large
arrays: one stream per 65,536-row chunk, SeedSequence([0xC5A2, workload, tensor, seq, chunk])),
so the same arguments always yield the same values on any host.

Value laws (the workloads this library is measured on):
  * main KV (post-RoPE latent, shared K=V): z ~ N(0,1) times a per-channel scale
    exp(U[ln 0.1, ln 8]), clipped to |x| <= 26, rounded to bf16 (RNE);
  * sliding-window KV: the same law, drawn separately per layer;
  * indexer keys and indexer queries: integers uniform in [-4, 4], stored as bf16;
  * indexer head weights: integers uniform in {1, 2, 3, 4}, stored as fp32;
  * attention queries: N(0,1) rounded to bf16.
The 26 bound is the visualisation page's caption on post-RoPE channel
magnitudes (it says at most about 26); the engineering article's section XI
bounds the same quantity by sqrt(512) ~ 22.6.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_ROOT = 0xC5A2

# tensor ids: one per kind of input, so streams never collide
T_KV = 1
T_KV_SIGMA = 2
T_IDX_K = 3
T_IDX_Q = 4
T_IDX_W = 5
T_Q = 6
T_SWA = 7
T_SWA_SIGMA = 8
T_LEN = 9
T_NEW_KV = 10
T_MISC = 11
T_SWA_NEW = 12   # the decode step's own window vector per layer

KV_CLIP = 26.0


def rng(workload: int, tensor: int, seq: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload, tensor, seq])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (round to nearest, ties to even); bit patterns.
    (In uint32 arithmetic: b + 0x7fff + 1 stays below 2^32 for every finite float.)"""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for building inputs and printing)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# bf16 bit patterns of the integers -4..4 (exact): lookup table for integer inputs
_INT_BF16 = f32_to_bf16_bits(np.arange(-4, 5, dtype=np.float32))


def channel_sigma(workload: int, tensor: int, dim: int, seq: int = 0) -> np.ndarray:
    r = rng(workload, tensor, seq)
    return np.exp(r.uniform(np.log(0.1), np.log(8.0), size=dim)).astype(np.float32)


CHUNK_ROWS = 1 << 16  # rows per independent stream of the large generators


def _chunked(n: int, fill) -> None:
    """Run fill(chunk_index, row_start, row_end) over fixed row chunks on a thread pool (numpy's
    generators release the GIL).  Each chunk has its own seeded stream, so the result does not
    depend on the number of threads."""
    chunks = [(c, s, min(n, s + CHUNK_ROWS)) for c, s in enumerate(range(0, n, CHUNK_ROWS))]
    if len(chunks) <= 1:
        for c in chunks:
            fill(*c)
        return
    workers = max(1, min(16, (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda c: fill(*c), chunks))


def kv_bf16(workload: int, tensor: int, n: int, dim: int, sigma: np.ndarray, seq: int = 0) -> np.ndarray:
    """[n, dim] bf16 bits: clip(N(0,1) * sigma_c, +-26), one stream per 65,536-row chunk."""
    out = np.empty((n, dim), dtype=np.uint16)

    def fill(c, s, e):
        r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload, tensor, seq, c])))
        z = r.standard_normal((e - s, dim), dtype=np.float32)
        z *= sigma[None, :]
        np.clip(z, -KV_CLIP, KV_CLIP, out=z)
        out[s:e] = f32_to_bf16_bits(z)

    _chunked(n, fill)
    return out


def int_bf16(workload: int, tensor: int, shape, lo: int = -4, hi: int = 4, seq: int = 0) -> np.ndarray:
    """Integers uniform in [lo, hi] (within [-4, 4]) as bf16 bits; 2-D arrays with more than one
    chunk of rows use one stream per 65,536-row chunk."""
    assert -4 <= lo <= hi <= 4
    shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
    if len(shape) == 2 and shape[0] > CHUNK_ROWS:
        out = np.empty(shape, dtype=np.uint16)

        def fill(c, s, e):
            r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload, tensor, seq, c])))
            v = r.integers(lo, hi + 1, size=(e - s, shape[1]), dtype=np.int8)
            out[s:e] = _INT_BF16[(v + 4).astype(np.intp)]

        _chunked(shape[0], fill)
        return out
    r = rng(workload, tensor, seq)
    v = r.integers(lo, hi + 1, size=shape, dtype=np.int8)
    return _INT_BF16[(v + 4).astype(np.intp)]


def int_weights(workload: int, tensor: int, shape, seq: int = 0) -> np.ndarray:
    r = rng(workload, tensor, seq)
    return r.integers(1, 5, size=shape).astype(np.float32)


def normal_bf16(workload: int, tensor: int, shape, seq: int = 0) -> np.ndarray:
    r = rng(workload, tensor, seq)
    return f32_to_bf16_bits(r.standard_normal(shape, dtype=np.float32))


def log_uniform_lengths(workload: int, n: int, lo: int, hi: int, seq: int = 0) -> np.ndarray:
    r = rng(workload, T_LEN, seq)
    return np.round(np.exp(r.uniform(np.log(lo), np.log(hi), size=n))).astype(np.int64)
