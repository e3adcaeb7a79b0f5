"""Seeded synthetic inputs for the CSA2 hot path.

This module only draws random numbers and stores them in the storage types the
path consumes (bf16 bit patterns as uint16, fp32 weights, int64 row offsets).
It holds none of the method's arithmetic: no quantisation, scoring, selection
or attention.  Both the HIP path and the CPU oracle are fed from here.

Every stream is numpy PCG64 seeded with SeedSequence([0xC5A2, workload, tensor, seq]),
so a (workload, tensor, seq) triple always yields the same values on any host.

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

KV_CLIP = 26.0


def rng(workload: int, tensor: int, seq: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, workload, tensor, seq])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for building inputs and printing)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# bf16 bit patterns of the integers -4..4 (exact): lookup table for integer inputs
_INT_BF16 = f32_to_bf16_bits(np.arange(-4, 5, dtype=np.float32))


def channel_sigma(workload: int, tensor: int, dim: int, seq: int = 0) -> np.ndarray:
    r = rng(workload, tensor, seq)
    return np.exp(r.uniform(np.log(0.1), np.log(8.0), size=dim)).astype(np.float32)


def kv_bf16(workload: int, tensor: int, n: int, dim: int, sigma: np.ndarray, seq: int = 0,
            chunk: int = 1 << 20) -> np.ndarray:
    """[n, dim] bf16 bits: clip(N(0,1) * sigma_c, +-26), generated in row chunks to bound host memory."""
    out = np.empty((n, dim), dtype=np.uint16)
    r = rng(workload, tensor, seq)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        z = r.standard_normal((e - s, dim), dtype=np.float32)
        z *= sigma[None, :]
        np.clip(z, -KV_CLIP, KV_CLIP, out=z)
        out[s:e] = f32_to_bf16_bits(z)
    return out


def int_bf16(workload: int, tensor: int, shape, lo: int = -4, hi: int = 4, seq: int = 0) -> np.ndarray:
    """Integers uniform in [lo, hi] (within [-4, 4]) as bf16 bits."""
    assert -4 <= lo <= hi <= 4
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
