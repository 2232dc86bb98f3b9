"""Brute-force helpers for the oracle pins (tests only).

They build logical K/V directly, page them into a pool with their own code and
compute dense attention with numpy, so they share nothing with the oracle's
gather or softmax."""
import math

import numpy as np

from workloads import f32_to_storage, poison_array, storage_to_f32


def draw(rng, shape, dtype):
    return f32_to_storage(rng.standard_normal(shape).astype(np.float32), dtype)


def to64(a, dtype):
    return storage_to_f32(a, dtype).astype(np.float64)


def page(logical_k, logical_v, bs, pool_blocks, rng, dtype, maxb=None):
    """Scatter per-sequence logical K/V ([ctx,H,D] each) into a poisoned pool
    of ``pool_blocks`` blocks at random places. Returns (kc, vc, tables)."""
    H, D = logical_k[0].shape[1:]
    need = [math.ceil(k.shape[0] / bs) for k in logical_k]
    maxb = maxb or max(1, max(need))
    ids = rng.permutation(pool_blocks)[: sum(need)]
    kc = poison_array((pool_blocks, H, bs, D), dtype)
    vc = poison_array((pool_blocks, H, bs, D), dtype)
    bt = np.full((len(logical_k), maxb), -1, np.int32)
    pos = 0
    for s, (k, v) in enumerate(zip(logical_k, logical_v)):
        for i in range(need[s]):
            b = int(ids[pos]); pos += 1
            bt[s, i] = b
            lo, hi = i * bs, min(k.shape[0], (i + 1) * bs)
            kc[b, :, : hi - lo, :] = np.transpose(k[lo:hi], (1, 0, 2))
            vc[b, :, : hi - lo, :] = np.transpose(v[lo:hi], (1, 0, 2))
    return kc, vc, bt


def dense_attention(q, K, V, scale, mask=None):
    """q [D], K/V [n,D] fp64; mask [n] bool of visible keys."""
    x = scale * (K @ q)
    if mask is not None:
        x = np.where(mask, x, -np.inf)
    w = np.exp(x - x.max())
    return (w @ V) / w.sum()
