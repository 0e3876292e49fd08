"""GPU parity of thought-adaptive eviction by segment (kvq_evict_tbe) with the
oracle ("ThinKV", Methodology, think-before-evict).

The hand-worked schedule of the oracle pins is checked on the GPU directly;
the five workload recipes at small sizes (many segments, long and short
runs, windows, ragged lengths) are compared with the oracle bit for bit, with
importances rounded to sixteenths so that ties are common; sequences with
mixed and single thought types, no candidates and whole-segment evictions
are covered; and the cache keeps working after the eviction (append into
the holes, attend again).
"""
import math

import numpy as np
import pytest

from eviction_kvq_decode_amd import workloads as wl
from helpers import small_geometry
from oracle import oracle as orc
from pairs import (SMALL_WORKLOADS, Pair, assert_attention_close, assert_mass_close, assert_same_cache,
                   log)

pytestmark = pytest.mark.gpu
HD = 128
R, E, T = 0, 1, 2


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _pair_from_tags(tag_rows, seed=11):
    """Oracle and GPU caches holding B sequences with the given tags."""
    from eviction_kvq_decode_amd import kvq

    B, n = len(tag_rows), max(len(t) for t in tag_rows)
    g = small_geometry(B, 8, 2, n_max=n)
    st = wl.empty_state(g, True)
    oc, gc = orc.OracleCache(g, st), kvq.Cache(g, st)
    rng = np.random.default_rng(seed)
    for i in range(n):
        k = rng.standard_normal((B, 2, HD)).astype(np.float16)
        v = rng.standard_normal((B, 2, HD)).astype(np.float16)
        tags = np.array([t[i] if i < len(t) else wl.TAG_SKIP for t in tag_rows], dtype=np.uint8)
        oc.append(k, v, tags)
        gc.append(_dev(k), _dev(v), _dev(tags))
    return oc, gc, g


def _kept(st, g, b):
    nb = int(st["n_blocks"][b])
    out = []
    for ent in st["table"][b * g.max_blocks: b * g.max_blocks + nb]:
        p, bid = int(ent >> 30), int(ent & 0x3FFFFFFF)
        m = int(st[f"mask{p}"][bid])
        out += [int(st[f"pos{p}"][bid * 16 + s]) for s in range(16) if (m >> s) & 1]
    return sorted(out)


TAGS = [R, R, R, R, E, E, E, T, T, R, R, R, R, R, T, E, E]
IMP = [0.1, 0.5, 0.3, 0.5, 0.2, 0.9, 0.1, 0.4, 0.6, 0.05, 0.7, 0.7, 0.2, 0.8, 0.3, 0.1, 0.2]


@pytest.mark.parametrize("args,expect", [
    ((2, 1, 1, 0, 0), [1, 5, 8, 10, 13, 14, 15, 16]),
    ((2, 1, 1, 2, 2), [0, 1, 3, 5, 8, 10, 13, 14, 15, 16]),
])
def test_hand_worked_schedule(args, expect):
    import torch

    oc, gc, g = _pair_from_tags([TAGS])
    imp = np.zeros((1, g.n_cap), dtype=np.float32)
    imp[0, : len(IMP)] = IMP
    gc.evict_tbe(_dev(imp), *args)
    torch.cuda.synchronize()
    assert _kept(gc.state_numpy(), g, 0) == expect
    oc.evict_tbe(imp, *args)
    assert_same_cache(oc, gc.state_numpy())


def test_mixed_sequences_against_oracle():
    """Long and short runs, a single-type sequence, a Transition-only one,
    an empty one, and one whose segments are all dropped to nothing."""
    import torch

    rng = np.random.default_rng(21)
    rows = [
        list(np.repeat(rng.integers(0, 3, 40), rng.integers(1, 12, 40))),   # many segments
        [R] * 150,                                                          # one segment
        [T] * 60,                                                           # Transition only
        [],                                                                 # empty
        [E] * 30 + [T] * 5 + [R] * 30 + [T] * 5 + [E] * 30 + [T] * 5,       # whole blocks emptied
        list(rng.integers(0, 3, 300)),                                      # short runs
    ]
    oc, gc, g = _pair_from_tags(rows)
    imp = (np.round(rng.exponential(1.0, (g.B, g.n_cap)) * 16) / 16).astype(np.float32)
    for args in [(8, 1, 2, 0, 0), (1, 0, 0, 0, 0), (4, 2, 1, 5, 9), (64, 4, 8, 3, 3)]:
        log(f"[gpu tbe] mixed sequences, (r0, r_min, t_keep, qw, rw) = {args}")
        gc.evict_tbe(_dev(imp), *args)
        oc.evict_tbe(imp, *args)
        torch.cuda.synchronize()
        assert gc.status == 0
        assert_same_cache(oc, gc.state_numpy())


def test_sequence_mask_against_oracle():
    """The eviction fires per sequence (where a Transition starts): masked-out
    sequences stay exactly as they are, including a block emptied before the
    call that an unmasked call would drop; the others match the oracle and
    the freed blocks are ranked over them in batch order."""
    import torch

    rng = np.random.default_rng(31)
    rows = [list(np.repeat(rng.integers(0, 3, 30), rng.integers(1, 12, 30))) for _ in range(6)]
    oc, gc, g = _pair_from_tags(rows)
    imp = (np.round(rng.exponential(1.0, (g.B, g.n_cap)) * 16) / 16).astype(np.float32)
    # sequence 2's first block emptied by hand on both sides
    st = gc.state_numpy()
    ent = int(st["table"][2 * g.max_blocks])
    pool, bid = ent >> 30, ent & 0x3FFFFFFF
    oc.st[f"mask{pool}"][bid] = 0
    gc.t[f"mask{pool}"].view(torch.int16)[bid] = 0
    for mask in ([1, 0, 0, 1, 1, 0], [0, 0, 0, 0, 0, 0], [0, 1, 1, 0, 0, 1]):
        sm = np.array(mask, dtype=np.uint8)
        log(f"[gpu tbe] sequence mask {mask}")
        before = gc.state_numpy()
        gc.evict_tbe(_dev(imp), 4, 1, 2, 0, 0, seq_mask=_dev(sm))
        oc.evict_tbe(imp, 4, 1, 2, 0, 0, seq_mask=sm)
        torch.cuda.synchronize()
        assert gc.status == 0
        after = gc.state_numpy()
        assert_same_cache(oc, after)
        for b in np.flatnonzero(sm == 0):
            row = slice(b * g.max_blocks, (b + 1) * g.max_blocks)
            assert np.array_equal(after["table"][row], before["table"][row])
            assert _kept(after, g, b) == _kept(before, g, b)


@pytest.fixture(scope="module", params=list(SMALL_WORKLOADS))
def pair(request):
    w = SMALL_WORKLOADS[request.param]
    log(f"[gpu tbe] building {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N=[{w.n_min},{w.n_max}]")
    p = Pair(w)
    p.fill()
    return p


def test_workload_tbe_bit_exact(pair):
    import torch

    w = pair.w
    rng = np.random.default_rng(4321 + w.wid)
    imp = (np.round(rng.exponential(1.0, (w.B, pair.g.n_cap)) * 16) / 16).astype(np.float32)
    qw, rw = (w.q_window, w.recent_window) if w.q_window or w.recent_window else (16, 32)
    pair.gc.evict_tbe(_dev(imp), 64, 2, 4, qw, rw)
    pair.oc.evict_tbe(imp, 64, 2, 4, qw, rw)
    torch.cuda.synchronize()
    assert_same_cache(pair.oc, pair.gc.state_numpy())
    # the cache keeps working: append into the holes, attend again
    pair.append_step(9)
    assert_same_cache(pair.oc, pair.gc.state_numpy())
    ref, got = pair.decode(wl.queries(w, 3))
    assert_attention_close(ref, got)
    assert_mass_close(pair.oc.st["seq_len"], ref, got)


def test_long_window_and_long_segments():
    """A 42k-token sequence of mixed runs beside one whose Reasoning and
    Execution segments (700 and 1300 candidates) have later Transitions:
    segments longer than 512 candidates are selected from values reloaded
    at every step rather than held in registers."""
    import torch

    rng = np.random.default_rng(31)
    n_long = 42_000
    long_row = list(np.repeat(rng.integers(0, 3, n_long // 20), rng.integers(1, 40, n_long // 20)))[:n_long]
    seg_row = [E] * 700 + [T] * 5 + [R] * 1300 + [T] * 5 + [E] * 20
    log(f"[gpu tbe] long window and segments: {len(long_row)} and {len(seg_row)} tokens")
    oc, gc, g = _pair_from_tags([long_row, seg_row])
    imp = (np.round(rng.exponential(1.0, (g.B, g.n_cap)) * 16) / 16).astype(np.float32)
    for args in [(64, 4, 8, 16, 32), (4, 1, 2, 0, 0)]:
        log(f"[gpu tbe] long window and segments, (r0, r_min, t_keep, qw, rw) = {args}")
        gc.evict_tbe(_dev(imp), *args)
        oc.evict_tbe(imp, *args)
        torch.cuda.synchronize()
        assert gc.status == 0
        assert_same_cache(oc, gc.state_numpy())
