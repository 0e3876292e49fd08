"""Pins of the oracle's cache path against the fp16 tokens that went in.

Tokens of all three thought types are appended through the oracle's cache
("ThinKV", Methodology, TBQ: group quantisation whose precision follows the
thought type; Continuous Thinking: typed blocks, slots addressed by
position).  For every valid slot the test finds the token by its position
and checks, for K and for V separately:

  - the stored (scale, zero) words and codes are those of quantising that
    token's own row group by group;
  - dequantising the slot gives back the fp16 input within half a
    quantisation step, with the step bounded from the input values alone
    (integer codec: (max - min) / (2^b - 1), rounded up to fp16; native
    codec: the format's own spacing at x / scale).

A slot that read another area's (scale, zero) words (V taking K's, or the
neighbouring token's) fails the bound, since the two rows are independent
draws.
"""
import numpy as np
import pytest

from oracle import oracle as orc

from helpers import fill, oracle_cache, small_geometry

HD = 128
GS = 32
BITS = (8, 4, 2)


def _tokens(rng, n, B, Hkv):
    # keys with a few large channels (as in the workloads), values plain
    k = rng.standard_normal((n, B, Hkv, HD))
    k[..., 5] *= 10.0
    k[..., 77] *= 10.0
    v = rng.standard_normal((n, B, Hkv, HD))
    # some constant groups and signed zeros
    k[3, 0, 0, 32:64] = 0.5
    v[4, 0, Hkv - 1, 0:32] = -0.0
    return k.astype(np.float16), v.astype(np.float16)


def _step_bound(x, bits):
    """Half a step above |x - x_hat| for one group, from the inputs only:
    step <= fp16 round-up of (max - min) / lv, and rint of the fp32 quotient
    adds at most lv * 2^-22 steps."""
    xf = x.astype(np.float64)
    lv = (1 << bits) - 1
    rng_ = xf.max() - xf.min()
    if rng_ == 0.0:
        return 0.0
    step = rng_ / lv * (1.0 + 2.0 ** -10) * (1.0 + 2.0 ** -22)
    return step * (0.5 + lv * 2.0 ** -22)


def _native_bound(x, pool):
    """|x - x_hat| bound for ThinKV's formats, from the inputs only.  With
    scale s <= amax / top * (1 + 2^-10) and y = x / s in [-top, top]:
    E4M3 (3 mantissa bits) is within 2^-4 |y| for normal y and 2^-10 in the
    subnormal range; E2M1 (values 0, .5, 1, 1.5, 2, 3, 4, 6) within |y| / 4
    above 1 and 1/4 below; ternary (rint in [-1, 1]) within 1/2."""
    xf = np.abs(x.astype(np.float64))
    amax = xf.max()
    if amax == 0.0:
        return np.zeros_like(xf)
    if pool == 0:
        s = amax / 448.0 * (1.0 + 2.0 ** -10)
        return 2.0 ** -4 * xf + 2.0 ** -10 * s
    if pool == 1:
        s = amax / 6.0 * (1.0 + 2.0 ** -10)
        return 0.25 * xf + 0.25 * s
    s = amax * (1.0 + 2.0 ** -10)
    return np.full_like(xf, 0.5 * s)


@pytest.mark.parametrize("codec", (0, 1))
def test_cache_round_trip_against_inputs(codec):
    rng = np.random.default_rng(40 + codec)
    B, Hkv, n = 3, 2, 180
    g = small_geometry(B, 4, Hkv, n, codec=codec)
    c = oracle_cache(g)
    k, v = _tokens(rng, n, B, Hkv)
    tags = rng.choice(3, size=(n, B)).astype(np.uint8)
    fill(c, k, v, tags)
    assert c.status == 0
    seen = 0
    for b in range(B):
        slots = c.valid_slots(b)
        assert sorted(s[3] for s in slots) == list(range(n))
        for pool, bid, slot, pos in slots:
            assert pool == tags[pos, b]
            bits = BITS[pool]
            for h in range(Hkv):
                kc, vc, ksz, vsz = c.slot_codes(pool, bid, h, slot)
                kh, vh = c.dequant_slot(pool, bid, h, slot)
                for x_in, codes, sz, xh in ((k[pos, b, h], kc, ksz, kh), (v[pos, b, h], vc, vsz, vh)):
                    grp = x_in.reshape(4, GS)
                    if codec == 1:
                        sc, zr, cq = orc.quantize_groups_native(grp, pool)
                    else:
                        sc, zr, cq = orc.quantize_groups(grp, bits)
                    assert np.array_equal(sz.reshape(4, 2)[:, 0], sc)
                    assert np.array_equal(sz.reshape(4, 2)[:, 1], zr)
                    assert np.array_equal(codes, cq.reshape(HD))
                    err = np.abs(xh - x_in.astype(np.float64)).reshape(4, GS)
                    for gi in range(4):
                        if codec == 1:
                            assert np.all(err[gi] <= _native_bound(grp[gi], pool)), (b, pos, h, gi)
                        else:
                            assert np.all(err[gi] <= _step_bound(grp[gi], bits)), (b, pos, h, gi)
                seen += 1
    assert seen == B * n * Hkv


def test_round_trip_catches_a_swapped_area():
    """The bound separates a slot's own V reconstruction from one built with
    its K (scale, zero) words: the check above has the power to catch that
    misread."""
    rng = np.random.default_rng(7)
    g = small_geometry(1, 2, 1, 40)
    c = oracle_cache(g)
    k, v = _tokens(rng, 40, 1, 1)
    tags = np.ones((40, 1), np.uint8)
    fill(c, k, v, tags)
    caught = 0
    for pool, bid, slot, pos in c.valid_slots(0):
        _, vc, ksz, _ = c.slot_codes(pool, bid, 0, slot)
        s = ksz.reshape(4, 2)[:, 0].view(np.float16).astype(np.float64)
        z = ksz.reshape(4, 2)[:, 1].view(np.float16).astype(np.float64)
        wrong = vc.reshape(4, GS) * s[:, None] + z[:, None]
        grp = v[pos, 0, 0].reshape(4, GS)
        err = np.abs(wrong - grp.astype(np.float64))
        caught += any(np.any(err[gi] > _step_bound(grp[gi], 4)) for gi in range(4))
    assert caught == 40
