"""Seeded synthetic inputs for the k8v4 cache and its attention.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantization, rotation or attention), so both the HIP
path and the CPU oracle can be fed from it.

Recipe (all draws from ``numpy.random.default_rng``):
  * values are standard normal, drawn in float32 and cast (round to nearest
    even) to the input dtype (float16, or float32 for the tiny case);
  * an optional set of outlier channels per KV head is multiplied by a
    factor (8x) on both K and V, for every token;
  * K/V are drawn per chunk of tokens from ``default_rng([seed, layer,
    chunk])``, K first then V, so any chunk can be regenerated on its own;
  * page tables are a seeded permutation of the physical pages (the first
    ``n_table`` entries of a permutation of ``n_pages``);
  * queries come from ``default_rng([seed, layer, 1_000_003, step])``.
"""
from __future__ import annotations

import math

import numpy as np

CHUNK = 8192          # tokens per generator chunk (and per append call in the workloads)
Q_STREAM = 1_000_003  # stream id that keeps queries apart from K/V chunks


def page_table(seed: int, n_table: int, n_pages: int, identity: bool = False) -> np.ndarray:
    """Logical page -> physical page, int32 [n_table], entries distinct."""
    if n_table > n_pages:
        raise ValueError("page table longer than the pool")
    if identity:
        return np.arange(n_table, dtype=np.int32)
    rng = np.random.default_rng([seed, 7_777_777])
    return rng.permutation(n_pages)[:n_table].astype(np.int32)


def outlier_channels(seed: int, n_kv_heads: int, head_dim: int, frac: float) -> np.ndarray:
    """[n_kv_heads][k] channel indices, k = ceil(frac * head_dim), sorted."""
    k = int(math.ceil(frac * head_dim))
    rng = np.random.default_rng([seed, 5_555_555])
    return np.stack([np.sort(rng.choice(head_dim, size=k, replace=False))
                     for _ in range(n_kv_heads)]).astype(np.int64)


def _normal(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return x.astype(dtype)


def kv_chunk(seed: int, layer: int, chunk: int, n: int, n_kv_heads: int, head_dim: int,
             dtype=np.float16, outliers: np.ndarray | None = None, outlier_scale: float = 8.0):
    """K, V for tokens [chunk*CHUNK, chunk*CHUNK + n): arrays [n][H][D] of dtype."""
    rng = np.random.default_rng([seed, layer, chunk])
    shape = (n, n_kv_heads, head_dim)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if outliers is not None:
        for g in range(n_kv_heads):
            k[:, g, outliers[g]] *= np.float32(outlier_scale)
            v[:, g, outliers[g]] *= np.float32(outlier_scale)
    return k.astype(dtype), v.astype(dtype)


def kv_tokens(seed: int, layer: int, pos0: int, n: int, n_kv_heads: int, head_dim: int,
              dtype=np.float16, outliers=None):
    """K, V for absolute token positions [pos0, pos0+n), assembled from chunks."""
    ks, vs = [], []
    p = pos0
    end = pos0 + n
    while p < end:
        c = p // CHUNK
        c0 = c * CHUNK
        k, v = kv_chunk(seed, layer, c, CHUNK, n_kv_heads, head_dim, dtype, outliers)
        a, b = p - c0, min(end, c0 + CHUNK) - c0
        ks.append(k[a:b])
        vs.append(v[a:b])
        p = c0 + b
    if not ks:
        shape = (0, n_kv_heads, head_dim)
        return np.zeros(shape, dtype), np.zeros(shape, dtype)
    return np.concatenate(ks), np.concatenate(vs)


def queries(seed: int, layer: int, step: int, rows: int, n_q_heads: int, head_dim: int,
            dtype=np.float16) -> np.ndarray:
    rng = np.random.default_rng([seed, layer, Q_STREAM, step])
    return _normal(rng, (rows, n_q_heads, head_dim), dtype)


# Workload shapes (head shape shared by every case).
N_Q_HEADS, N_KV_HEADS, HEAD_DIM = 16, 2, 256

WORKLOADS = {
    "tiny_roundtrip": dict(ctx=1024, page_size=16, n_pages=64, dtype="float32", seed=0,
                           outlier_frac=0.0),
    "decode_32k": dict(ctx=32768, page_size=256, n_pages=256, dtype="float16", seed=2,
                       outlier_frac=0.01),
    "decode_118k_48l": dict(ctx=118750, page_size=256, n_pages=464, dtype="float16", seed=3,
                            layers=48, outlier_frac=0.0),
    "verify_240k": dict(ctx=240000, page_size=256, n_pages=1024, dtype="float16", seed=4,
                        n_q=5, outlier_frac=0.0),
    "prefill_chunk_240k": dict(ctx=240000, page_size=256, n_pages=1024, dtype="float16", seed=5,
                               n_new=8192, outlier_frac=0.0),
}


# ---------------------------------------------------------------- device-side draws
# For benchmark-scale fills (gigabytes of K/V) the same recipe is drawn on the
# GPU with torch's Philox generator: standard normal fp32, cast to fp16,
# one generator per (seed, layer, chunk) seeded with seed_of(...).  These
# values differ from the numpy stream above; they only feed timing runs.

def seed_of(seed: int, layer: int, chunk: int) -> int:
    return (seed * 1_000_003 + layer) * 1_000_033 + chunk


def kv_chunk_device(seed: int, layer: int, chunk: int, n: int, n_kv_heads: int, head_dim: int,
                    device, dtype=None, outliers=None, outlier_scale: float = 8.0):
    """outliers: optional [n_kv_heads][k] channel indices scaled on K and V."""
    import torch
    dtype = dtype or torch.float16
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(seed, layer, chunk))
    k = torch.randn((n, n_kv_heads, head_dim), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((n, n_kv_heads, head_dim), generator=gen, device=device, dtype=torch.float32)
    if outliers is not None:
        for g in range(n_kv_heads):
            ch = torch.as_tensor(outliers[g], device=device)
            k[:, g, ch] *= outlier_scale
            v[:, g, ch] *= outlier_scale
    return k.to(dtype), v.to(dtype)


def queries_device(seed: int, layer: int, step: int, rows: int, n_q_heads: int, head_dim: int,
                   device, dtype=None):
    import torch
    dtype = dtype or torch.float16
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_of(seed, layer, Q_STREAM + step))
    return torch.randn((rows, n_q_heads, head_dim), generator=gen, device=device,
                       dtype=torch.float32).to(dtype)
