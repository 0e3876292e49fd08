"""Pins of the oracle's decode attention, attention mass and importance.

Scaled dot-product attention over the cached K/V ("Back from the Future",
Problem Statement), mass = attention weight a token receives summed over
query heads ("Thought-Aware KV Cache Compaction ...", sections 1 and 2.B),
importance accumulated H2O-style with a decay.
"""
import math

import numpy as np
import pytest
import torch

from helpers import dense_kv, fill, oracle_cache, random_tokens, small_geometry

HD = 128
SM = 1.0 / math.sqrt(HD)


def _build(rng, B=2, Hq=8, Hkv=2, n=300, tag_p=(0.3, 0.4, 0.3), identity=False, seed_key=(0,)):
    g = small_geometry(B, Hq, Hkv, n)
    c = oracle_cache(g, identity_ids=identity, seed_key=seed_key)
    k, v = random_tokens(rng, B, Hkv, n)
    tags = rng.choice(3, size=(n, B), p=tag_p).astype(np.uint8)
    fill(c, k, v, tags)
    return g, c, (k, v, tags)


def test_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(0)
    g, c, _ = _build(rng, n=300)
    q = rng.standard_normal((g.B, g.Hq, HD)).astype(np.float16)
    out, mass, _ = c.decode(q, SM)
    G = g.Hq // g.Hkv
    for b in range(g.B):
        ref_mass = np.zeros(g.n_cap)
        for h in range(g.Hq):
            K, V, pos = dense_kv(c, b, h // G)
            qt = torch.from_numpy(q[b, h].astype(np.float64))[None, None, None, :]
            o = torch.nn.functional.scaled_dot_product_attention(
                qt, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None], scale=SM)
            assert np.allclose(out[b, h], o[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)
            p = torch.softmax(torch.from_numpy(K) @ qt[0, 0, 0] * SM, dim=0).numpy()
            np.add.at(ref_mass, pos, p)
        assert np.allclose(mass[b], ref_mass, rtol=1e-12, atol=1e-15)
        assert math.isclose(mass[b].sum(), g.Hq, rel_tol=1e-12)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    g = small_geometry(1, 8, 2, 200)
    c = oracle_cache(g)
    n = 200
    kvec = rng.standard_normal((1, 2, HD)).astype(np.float16)
    k = np.broadcast_to(kvec, (n, 1, 2, HD)).copy()
    v = rng.standard_normal((n, 1, 2, HD)).astype(np.float16)
    tags = rng.choice(3, size=(n, 1)).astype(np.uint8)
    # identical fp16 rows quantise to identical codes only within one bit
    # width, so give every token the same type
    tags[:] = 1
    fill(c, k, v, tags)
    q = rng.standard_normal((1, 8, HD)).astype(np.float16)
    out, mass, _ = c.decode(q, SM)
    for h in range(8):
        _, V, pos = dense_kv(c, 0, h // 4)
        assert np.allclose(out[0, h], V.mean(axis=0), rtol=1e-12, atol=1e-14)
        # and the mean of the fp16 inputs, within half a 4-bit step per
        # group (bounded from the inputs: (max - min) / 15 rounded up to fp16)
        vin = v[:, 0, h // 4].astype(np.float64).reshape(n, 4, 32)
        half_step = (vin.max(axis=2) - vin.min(axis=2)) / 15 * (1 + 2.0 ** -10) * (0.5 + 2.0 ** -18)
        bound = np.repeat(half_step.mean(axis=0), 32)
        assert np.all(np.abs(out[0, h] - vin.reshape(n, 128).mean(axis=0)) <= bound + 1e-12)
    assert np.allclose(mass[0, :n], 8.0 / n, rtol=1e-12)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(2)
    g = small_geometry(1, 4, 1, 100)
    c = oracle_cache(g)
    n, j = 100, 37
    q = rng.standard_normal((1, 4, HD)).astype(np.float16)
    k, v = random_tokens(rng, 1, 1, n)
    # token j's key points along the mean query direction, score gap >> 40
    qm = q[0].astype(np.float32).mean(axis=0)
    k[j, 0, 0] = (40.0 * qm / np.abs(qm).max()).astype(np.float16)
    tags = rng.choice(3, size=(n, 1)).astype(np.uint8)
    tags[j] = 0                                   # 8-bit keeps the direction
    fill(c, k, v, tags)
    out, mass, _ = c.decode(q, SM)
    K, V, pos = dense_kv(c, 0, 0)
    jj = int(np.where(pos == j)[0][0])
    s = (K @ q[0].astype(np.float64).T) * SM       # [n][4]
    gap = s[jj] - np.delete(s, jj, axis=0).max(axis=0)
    assert gap.min() > 40
    for h in range(4):
        assert np.allclose(out[0, h], V[jj], rtol=0, atol=1e-12 * np.abs(V).max() + 1e-15)
    assert abs(mass[0, j] - 4.0) < 1e-12


def test_probabilities_and_mass_sum():
    rng = np.random.default_rng(3)
    g, c, _ = _build(rng, B=3, Hq=12, Hkv=3, n=257)
    q = rng.standard_normal((g.B, g.Hq, HD)).astype(np.float16)
    _, mass, _ = c.decode(q, SM)
    for b in range(g.B):
        assert math.isclose(mass[b].sum(), g.Hq, rel_tol=1e-12)
        assert np.all(mass[b] >= 0)
        assert not mass[b, 257:].any()


def test_layout_invariance():
    """Physical block ids and table order do not change the result."""
    rng = np.random.default_rng(4)
    n = 180
    g = small_geometry(2, 8, 2, n)
    k, v = random_tokens(rng, 2, 2, n)
    tags = rng.choice(3, size=(n, 2)).astype(np.uint8)
    q = rng.standard_normal((2, 8, HD)).astype(np.float16)
    a = oracle_cache(g, identity_ids=True)
    b = oracle_cache(g, identity_ids=False, seed_key=(7,))
    fill(a, k, v, tags)
    fill(b, k, v, tags)
    assert not np.array_equal(a.st["table"], b.st["table"])
    oa, ma, _ = a.decode(q, SM)
    ob, mb, _ = b.decode(q, SM)
    assert np.array_equal(oa, ob) and np.array_equal(ma, mb)
    # reverse sequence 0's table row: same values up to summation order
    row = b.st["table"][: b.st["n_blocks"][0]]
    b.st["table"][: b.st["n_blocks"][0]] = row[::-1].copy()
    oc, mc, _ = b.decode(q, SM)
    assert np.allclose(oc, ob, rtol=1e-12, atol=1e-14) and np.allclose(mc, mb, rtol=1e-12, atol=1e-16)


def test_holes_equal_dense_cache_of_survivors():
    """Attending over evicted holes equals attending over a cache that only
    ever held the surviving tokens."""
    rng = np.random.default_rng(5)
    n = 240
    g = small_geometry(1, 8, 2, n)
    k, v = random_tokens(rng, 1, 2, n)
    tags = rng.choice(3, size=(n, 1)).astype(np.uint8)
    keep = rng.random(n) < 0.45
    holey = oracle_cache(g)
    fill(holey, k, v, tags)
    imp = np.zeros((1, g.n_cap), dtype=np.float32)
    imp[0, :n] = keep
    holey.evict(imp, np.array([keep.sum()], dtype=np.int32), 0, 0)
    assert sorted(s[3] for s in holey.valid_slots(0)) == list(np.where(keep)[0])
    dense = oracle_cache(g)
    fill(dense, k[keep], v[keep], tags[keep])
    q = rng.standard_normal((1, 8, HD)).astype(np.float16)
    oh, mh, _ = holey.decode(q, SM)
    od, md, _ = dense.decode(q, SM)
    assert np.allclose(oh, od, rtol=1e-12, atol=1e-14)
    assert np.allclose(mh[0, np.where(keep)[0]], md[0, : keep.sum()], rtol=1e-12, atol=1e-16)
    assert not mh[0, np.where(~keep)[0]].any()


def test_importance_recurrence_closed_form():
    rng = np.random.default_rng(6)
    g, c, _ = _build(rng, B=1, Hq=8, Hkv=2, n=150)
    q = rng.standard_normal((1, 8, HD)).astype(np.float16)
    I0 = rng.exponential(0.05, size=(1, g.n_cap)).astype(np.float32)
    I = I0.copy()
    steps, decay = 12, 0.9
    for _ in range(steps):
        _, m, I = c.decode(q, SM, importance=I, decay=decay)
    valid = np.zeros(g.n_cap, bool)
    valid[:150] = True
    closed = decay ** steps * I0[0].astype(np.float64) + m[0] * (1 - decay ** steps) / (1 - decay)
    assert np.allclose(I[0, valid], closed[valid], rtol=2e-6, atol=1e-9)
    assert np.array_equal(I[0, ~valid], I0[0, ~valid])
