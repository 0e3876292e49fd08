"""Pins of the oracle's fp16 conversion, quantiser and cache format.

Checked against numpy's IEEE binary16 conversion, closed forms of min/max
group quantisation ("ThinKV", Methodology, TBQ: group quantisation by
thought type) and exhaustive pack/unpack round trips.
"""
import numpy as np
import pytest

from oracle import oracle as orc

from helpers import oracle_cache, small_geometry

BITS = (8, 4, 2)


def test_half_to_double_exhaustive():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.half_to_double(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_float_to_half_matches_numpy():
    rng = np.random.default_rng(1)
    # random floats across the whole binary16 range and beyond
    e = rng.uniform(-30, 17, size=400_000)
    f = (np.sign(rng.standard_normal(e.size)) * np.exp2(e)).astype(np.float32)
    # exact halfway points between adjacent halves (ties), incl. subnormals
    hb = np.arange(0, 0x7BFF, dtype=np.uint32).astype(np.uint16)
    lo = hb.view(np.float16).astype(np.float64)
    hi = (hb + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)      # exact in fp32
    edge = np.array([0.0, -0.0, 65504, 65519.996, 65520, 65536, 1e-8, 2.9802322e-08,
                     5.9604645e-08, 6.1035156e-05, np.inf, -np.inf], dtype=np.float32)
    for x in (f, mid, -mid, edge):
        with np.errstate(over="ignore"):
            ref = x.astype(np.float16).view(np.uint16)
        assert np.array_equal(orc.float_to_half(x), ref)


def _groups(rng, n, scale=1.0):
    return (rng.standard_normal((n, 32)) * scale).astype(np.float16)


@pytest.mark.parametrize("bits", BITS)
def test_quantiser_round_trip_bound(bits):
    rng = np.random.default_rng(bits)
    lv = (1 << bits) - 1
    x = np.concatenate([_groups(rng, 4000), _groups(rng, 1000, 10.0), _groups(rng, 500, 1e-3),
                        _groups(rng, 200, 3000.0)])
    sc, zr, codes = orc.quantize_groups(x, bits)
    s = sc.view(np.float16).astype(np.float64)
    z = zr.view(np.float16).astype(np.float64)
    xh = codes * s[:, None] + z[:, None]
    err = np.abs(x.astype(np.float64) - xh)
    # rint puts every code within 1/2 step; fp32 rounding of the quotient
    # adds at most lv * 2^-22 steps
    bound = s[:, None] * (0.5 + lv * 2.0 ** -22)
    assert np.all(err <= bound)
    assert codes.max() <= lv
    # zero is the group minimum, exactly
    assert np.array_equal(z, x.astype(np.float64).min(axis=1))


@pytest.mark.parametrize("bits", BITS)
def test_scale_is_least_half_above_range(bits):
    rng = np.random.default_rng(10 + bits)
    lv = (1 << bits) - 1
    x = np.concatenate([_groups(rng, 3000), _groups(rng, 300, 1e-4)])
    sc, zr, _ = orc.quantize_groups(x, bits)
    xf = x.astype(np.float32)
    s32 = (xf.max(axis=1) - xf.min(axis=1)) / np.float32(lv)
    s = sc.view(np.float16).astype(np.float64)
    assert np.all(s >= s32.astype(np.float64))
    nz = sc > 0
    prev = (sc[nz] - 1).astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.all(prev < s32[nz].astype(np.float64))


@pytest.mark.parametrize("bits", BITS)
def test_ramp_codes_are_exact(bits):
    lv = (1 << bits) - 1
    step = 2.0 ** -4
    idx = np.linspace(0, lv, 32).round().astype(np.int64)   # covers 0 and lv
    x = (-1.0 + idx * step).astype(np.float16)[None, :]
    sc, zr, codes = orc.quantize_groups(x, bits)
    assert sc.view(np.float16)[0] == np.float16(step)
    assert zr.view(np.float16)[0] == np.float16(-1.0)
    assert np.array_equal(codes[0], idx)


@pytest.mark.parametrize("bits", BITS)
def test_constant_and_signed_zero_groups(bits):
    x = np.full((1, 32), 0.75, dtype=np.float16)
    sc, zr, codes = orc.quantize_groups(x, bits)
    assert sc[0] == 0 and zr.view(np.float16)[0] == np.float16(0.75) and not codes.any()
    z = np.zeros((1, 32), dtype=np.float16)
    z[0, ::2] = np.float16(-0.0)
    sc, zr, codes = orc.quantize_groups(z, bits)
    assert sc[0] == 0 and zr[0] == 0 and not codes.any()     # -0 stored as +0
    y = np.zeros((1, 32), dtype=np.float16)
    y[0, 0] = np.float16(-0.0)
    y[0, 5] = np.float16(1.0)
    sc, zr, codes = orc.quantize_groups(y, bits)
    assert zr[0] == 0


@pytest.mark.parametrize("bits", BITS)
def test_codes_monotone_in_x(bits):
    rng = np.random.default_rng(20 + bits)
    x = _groups(rng, 2000)
    _, _, codes = orc.quantize_groups(x, bits)
    order = np.argsort(x.astype(np.float64), axis=1, kind="stable")
    c_sorted = np.take_along_axis(codes.astype(np.int64), order, axis=1)
    assert np.all(np.diff(c_sorted, axis=1) >= 0)


@pytest.mark.parametrize("bits", BITS)
def test_code_positions_are_a_bijection(bits):
    area = 256 * bits * 8            # bits in the K (or V) code area of one region
    kpos = np.array([[orc.k_bit_offset(bits, t, d) for d in range(128)] for t in range(16)])
    vpos = np.array([[orc.v_bit_offset(bits, t, d) for d in range(128)] for t in range(16)])
    for pos in (kpos, vpos):
        assert np.all(pos % bits == 0)
        assert np.array_equal(np.sort(pos.ravel()), np.arange(0, area, bits))
    # a K row is contiguous per token
    assert np.array_equal(kpos.min(axis=1), np.arange(16) * 128 * bits)


@pytest.mark.parametrize("bits", BITS)
def test_pack_unpack_exhaustive(bits):
    pool = {8: 0, 4: 1, 2: 2}[bits]
    g = small_geometry(1, 2, 2, 64)
    c = oracle_cache(g, identity_ids=True)
    lv = (1 << bits) - 1
    rng = np.random.default_rng(bits)
    written = {}
    for h in range(2):
        for t in range(16):
            kc = (np.arange(128) + 7 * t + h) % (lv + 1)      # every code value at every d
            vc = rng.integers(0, lv + 1, 128)
            c.put_slot_codes(pool, 3, h, t, kc, vc)
            written[(h, t)] = (kc, vc)
    for (h, t), (kc, vc) in written.items():
        rk, rv, _, _ = c.slot_codes(pool, 3, h, t)
        assert np.array_equal(rk, kc) and np.array_equal(rv, vc)
    # neighbouring blocks untouched
    rb = orc.region_bytes(bits)
    kv = c.st[f"kv{pool}"]
    assert not kv[: 3 * 2 * rb].any() and not kv[4 * 2 * rb:].any()
