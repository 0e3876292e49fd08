"""Pins of the oracle's native formats ("ThinKV", Methodology, TBQ: FP8 for
Reasoning, 4-bit FP for Execution, ternary for Transition tokens).

E4M3 and E2M1 are the OCP 8- and 4-bit floating-point formats.  E4M3 is
checked exhaustively against torch's float8_e4m3fn, in both directions.
E2M1 is checked against its eight magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6},
its round-to-nearest-even ties and a brute-force nearest search.  Then come
the group quantiser's scale, error bounds, ternary thresholds and
degenerate groups, and attention over a native-format cache against torch's
SDPA on the dequantised tensors.
"""
import math

import numpy as np
import torch

from helpers import dense_kv, fill, oracle_cache, random_tokens, small_geometry
from oracle import oracle as orc

HD = 128
SM = 1.0 / math.sqrt(HD)
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_decode_matches_torch_exhaustively():
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.native_values(0, codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]  # the format's NaNs, never produced
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch():
    rng = np.random.default_rng(0)
    y = np.concatenate([
        rng.standard_normal(100000) * 100, rng.standard_normal(100000) * 0.01,
        (rng.integers(-448 * 64, 448 * 64, 20000) / 64.0),     # many exact ties
        [448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 0.0],
    ]).astype(np.float32)
    y = np.clip(y, -448.0, 448.0)
    ours = orc.mini_encode(y, 0)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # a negative that rounds to a zero magnitude is stored as +0 here
    neg_zero = (ref == 0x80) & (ours == 0)
    assert np.array_equal(ours[~neg_zero], ref[~neg_zero])
    # saturation above the largest magnitude instead of NaN
    assert orc.mini_encode(np.array([500.0, -1e6], dtype=np.float32), 0).tolist() == [0x7E, 0xFE]


def test_e2m1_values_ties_and_nearest():
    assert orc.native_values(1, np.arange(8, dtype=np.uint8)).tolist() == E2M1
    assert orc.native_values(1, np.arange(8, 16, dtype=np.uint8)).tolist() == [-v for v in E2M1]
    # ties go to the even code: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert orc.native_values(1, orc.mini_encode(ties, 1)).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert orc.mini_encode(np.array([7.0, -100.0], dtype=np.float32), 1).tolist() == [7, 15]
    rng = np.random.default_rng(1)
    y = rng.uniform(-6, 6, 20000).astype(np.float32)
    got = orc.native_values(1, orc.mini_encode(y, 1))
    grid = np.array(E2M1)
    for yi, gi in zip(y, got):
        d = np.abs(grid - abs(yi))
        assert abs(gi) in grid[d == d.min()] and (gi == 0 or np.sign(gi) == np.sign(yi))


def _groups(rng, n, scale=1.0):
    return (rng.standard_normal((n, 32)) * scale).astype(np.float16)


def test_scale_is_least_fp16_above_amax_over_top():
    rng = np.random.default_rng(2)
    x = np.concatenate([_groups(rng, 300), _groups(rng, 300, 0.001), _groups(rng, 300, 300.0)])
    for pool, top in [(0, 448.0), (1, 6.0), (2, 1.0)]:
        sc, zr, _ = orc.quantize_groups_native(x, pool)
        s = sc.view(np.float16).astype(np.float64)
        amax = np.abs(x.astype(np.float64)).max(axis=1)
        want = (amax.astype(np.float32) / np.float32(top)).astype(np.float64)
        below = np.nextafter(s.astype(np.float16), np.float16(0)).astype(np.float64)
        assert np.all(s >= want) and np.all(below < want)
        z = zr.view(np.float16).astype(np.float64)
        assert np.array_equal(z, -s if pool == 2 else np.zeros_like(s))


def test_round_trip_error_bounds():
    rng = np.random.default_rng(3)
    x = np.concatenate([_groups(rng, 500), _groups(rng, 100, 20.0)])
    xf = x.astype(np.float64)
    for pool in (0, 1):
        sc, zr, codes = orc.quantize_groups_native(x, pool)
        s = sc.view(np.float16).astype(np.float64)[:, None]
        xh = orc.native_values(pool, codes) * s
        # half a step: 2^-(M+1) relative for normals, half the subnormal step
        # (2^-10 or 2^-1 of the scale) absolute, plus the division rounding
        rel, sub = (2.0 ** -4, 2.0 ** -10) if pool == 0 else (2.0 ** -2, 2.0 ** -1)
        err = np.abs(xh - xf)
        assert np.all(err <= rel * np.abs(xf) + sub * s + 1e-6 * np.abs(xf))
        # the largest element lands within a step of the top of the format
        top = 448.0 if pool == 0 else 6.0
        assert np.all(np.abs(orc.native_values(pool, codes)).max(axis=1) >= top * (0.875 if pool == 0 else 0.66))
    sc, zr, codes = orc.quantize_groups_native(x, 2)
    s = sc.view(np.float16).astype(np.float64)[:, None]
    t = codes.astype(np.float64) - 1.0
    assert set(np.unique(codes)) <= {0, 1, 2}
    assert np.array_equal(t, np.clip(np.round(xf / s), -1, 1))  # ties to even (0.5 -> 0)
    assert np.all(np.abs(t * s - xf) <= s / 2 + 1e-12)


def test_sign_symmetry_and_degenerate_groups():
    rng = np.random.default_rng(4)
    x = _groups(rng, 200)
    for pool in (0, 1):
        _, _, c1 = orc.quantize_groups_native(x, pool)
        _, _, c2 = orc.quantize_groups_native(-x, pool)
        v1, v2 = orc.native_values(pool, c1), orc.native_values(pool, c2)
        assert np.array_equal(v1, -v2)
    z = np.zeros((2, 32), dtype=np.float16)
    z[1] = -0.0
    for pool, zero_code in [(0, 0), (1, 0), (2, 1)]:
        sc, zr, codes = orc.quantize_groups_native(z, pool)
        assert sc.tolist() == [0, 0] and zr.tolist() == [0, 0] and np.all(codes == zero_code)


def test_native_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(5)
    g = small_geometry(2, 8, 2, 300, codec=1)
    c = oracle_cache(g)
    k, v = random_tokens(rng, 2, 2, 300)
    tags = rng.choice(3, size=(300, 2)).astype(np.uint8)
    fill(c, k, v, tags)
    q = rng.standard_normal((2, 8, HD)).astype(np.float16)
    out, mass, _ = c.decode(q, SM)
    for b in range(2):
        ref_mass = np.zeros(g.n_cap)
        for h in range(8):
            K, V, pos = dense_kv(c, b, h // 4)
            qt = torch.from_numpy(q[b, h].astype(np.float64))[None, None, None, :]
            o = torch.nn.functional.scaled_dot_product_attention(
                qt, torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None], scale=SM)
            assert np.allclose(out[b, h], o[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)
            ref_mass[pos] += torch.softmax(torch.from_numpy(K) @ qt[0, 0, 0] * SM, dim=0).numpy()
        assert np.allclose(mass[b], ref_mass, rtol=1e-12, atol=1e-15)
    # and the dequantised cache is the native formats' reconstruction of the inputs
    K, V, pos = dense_kv(c, 0, 0)
    order = np.argsort(pos)
    kin = k[pos[order], 0, 0].astype(np.float64)
    assert np.max(np.abs(K[order] - kin)) < 0.6 * np.abs(kin).max()
