"""Shared test plumbing: build caches from the seeded workloads."""
from __future__ import annotations

import math

import numpy as np

from eviction_kvq_decode_amd import workloads as wl
from oracle import oracle as orc

HD = 128
BLK = 16


def small_geometry(B, Hq, Hkv, n_max, pool_blocks=None, max_blocks=None, n_cap=None, codec=0):
    if max_blocks is None:
        max_blocks = math.ceil(n_max / BLK) + 8
    if pool_blocks is None:
        pb = B * max_blocks
        pool_blocks = (pb, pb, pb)
    if n_cap is None:
        n_cap = n_max + 64
    return wl.Geometry(B, Hq, Hkv, max_blocks, n_cap, tuple(pool_blocks), codec)


def oracle_cache(g, identity_ids=False, seed_key=(0,)):
    return orc.OracleCache(g, wl.empty_state(g, identity_ids, seed_key))


def random_tokens(rng, B, Hkv, n=1, scale=1.0):
    k = (rng.standard_normal((n, B, Hkv, HD)) * scale).astype(np.float16)
    v = rng.standard_normal((n, B, Hkv, HD)).astype(np.float16)
    return k, v


def fill(cache, k, v, tags):
    """Append tokens in lock-step: k, v [n][B][Hkv][128], tags [n][B]."""
    for i in range(k.shape[0]):
        cache.append(k[i], v[i], tags[i])


def dense_kv(cache, b, h):
    """Dequantised K, V [n_valid][128] and positions, in table order."""
    slots = cache.valid_slots(b)
    K = np.empty((len(slots), HD))
    V = np.empty((len(slots), HD))
    pos = np.empty(len(slots), dtype=np.int64)
    for i, (p, bid, s, ps) in enumerate(slots):
        K[i], V[i] = cache.dequant_slot(p, bid, h, s)
        pos[i] = ps
    return K, V, pos
