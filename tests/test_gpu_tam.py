"""GPU parity of thought-aware segment budgets (kvq_evict_tam) with the
oracle ("Thought-Aware KV Cache Compaction ... (TAM)", section 2: segments,
budgets proportional to sqrt(w) n, pivotal tokens).

The hand-worked pins of the oracle run on the GPU; mixed sequences under
several (pivot_c, min_seg, window) settings, every small workload (followed
by an append into the holes and a decode) and a sequence with segments of
hundreds of candidates and pivotal tokens among them are compared with the
oracle bit for bit.  Scores are multiples of 1/16, so ties are common.
"""
import numpy as np
import pytest

from eviction_kvq_decode_amd import workloads as wl
from helpers import small_geometry
from oracle import oracle as orc
from pairs import SMALL_WORKLOADS, Pair, assert_attention_close, assert_mass_close, assert_same_cache, log

pytestmark = pytest.mark.gpu
HD = 128
R, E, T = 0, 1, 2
INF = float("inf")


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _pair_from_tags(tag_rows, seed=11):
    from eviction_kvq_decode_amd import kvq

    B, n = len(tag_rows), max(1, max(len(t) for t in tag_rows))
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


def _run_both(oc, gc, g, scores, keep, pivot_c, min_seg, qw, rw):
    import torch

    kk = np.broadcast_to(np.asarray(keep, dtype=np.int32), (g.B,)).copy()
    gc.evict_tam(_dev(scores), _dev(kk), pivot_c, min_seg, qw, rw)
    oc.evict_tam(scores, kk, pivot_c, min_seg, qw, rw)
    torch.cuda.synchronize()
    assert gc.status == 0


HAND = [
    # tags, scores, (keep, pivot_c, min_seg, qw, rw), kept positions
    ([R] * 8 + [E] * 8, [3, 5] * 4 + [0.5, 1.5] * 4, (6, INF, 1, 0, 0), [1, 3, 5, 7, 9, 11]),
    ([R] * 2 + [E] * 10 + [T] * 10, [100, 100] + [0.5, 1.5] * 10, (8, INF, 1, 0, 0),
     [0, 1, 3, 5, 7, 13, 15, 17]),
    ([R] * 10, [1] * 9 + [11], (4, 3.0, 1, 0, 0), [0, 1, 2, 9]),
    ([R] * 8 + [E] * 8, [1] * 7 + [57] + [8] * 8, (9, 3.0, 1, 0, 0), [0, 1, 2, 7, 8, 9, 10, 11, 12]),
    ([R, R, R, E, R, R, R, E, E, E], [9, 9, 9, 1, 4, 4, 4, 2, 2, 2], (5, INF, 2, 0, 0), [0, 1, 4, 7, 8]),
    ([R, R, R, E, R, R, R, E, E, E], [9, 9, 9, 1, 4, 4, 4, 2, 2, 2], (5, INF, 1, 0, 0), [0, 1, 4, 7, 8]),
    ([R, R, R, E, R, R, R, E, E, E], [9, 9, 9, 1, 4, 4, 4, 2, 2, 2], (5, INF, 4, 0, 0), [0, 1, 2, 4, 5]),
]


@pytest.mark.parametrize("tags,scores,args,expect", HAND)
def test_hand_worked_budgets(tags, scores, args, expect):
    oc, gc, g = _pair_from_tags([tags])
    sc = np.zeros((1, g.n_cap), dtype=np.float32)
    sc[0, : len(scores)] = scores
    _run_both(oc, gc, g, sc, *args)
    assert _kept(gc.state_numpy(), g, 0) == expect
    assert_same_cache(oc, gc.state_numpy())


def test_mixed_sequences_against_oracle():
    """Many segments, one segment, Transition only, empty, short runs, and
    segments of hundreds of candidates (the LDS-histogram selection) with
    pivotal tokens among them."""
    rng = np.random.default_rng(23)
    rows = [
        list(np.repeat(rng.integers(0, 3, 40), rng.integers(1, 12, 40))),
        [R] * 150,
        [T] * 60,
        [],
        list(rng.integers(0, 3, 300)),
        [E] * 700 + [T] * 5 + [R] * 1300 + [T] * 5 + [E] * 20,
    ]
    sc = None
    for args in [(64, INF, 1, 0, 0), (64, 4.0, 1, 0, 0), (200, 8.0, 8, 5, 9), (10, 2.0, 32, 3, 3),
                 (0, 6.0, 1, 0, 0), (5000, INF, 1, 0, 0)]:
        log(f"[gpu tam] mixed sequences, (keep, c, min_seg, qw, rw) = {args}")
        oc, gc, g = _pair_from_tags(rows)
        if sc is None:
            sc = (np.round(rng.exponential(1.0, (g.B, g.n_cap)) * 16) / 16).astype(np.float32)
            sc[:, ::97] = 40.0  # a few pivotal tokens at every c used below
        _run_both(oc, gc, g, sc, *args)
        assert_same_cache(oc, gc.state_numpy())


@pytest.fixture(scope="module", params=list(SMALL_WORKLOADS))
def pair(request):
    w = SMALL_WORKLOADS[request.param]
    log(f"[gpu tam] building {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N=[{w.n_min},{w.n_max}]")
    p = Pair(w)
    p.fill()
    return p


def test_workload_tam_bit_exact(pair):
    import torch

    w = pair.w
    rng = np.random.default_rng(5150 + w.wid)
    sc = (np.round(rng.exponential(1.0, (w.B, pair.g.n_cap)) * 16) / 16).astype(np.float32)
    keep = np.maximum(16, (pair.oc.st["seq_len"].astype(np.int64) // 4)).astype(np.int32)
    qw, rw = (w.q_window, w.recent_window) if w.q_window or w.recent_window else (16, 32)
    kk = _dev(keep)
    pair.gc.evict_tam(_dev(sc), kk, 3.0, 4, qw, rw)
    pair.oc.evict_tam(sc, keep, 3.0, 4, qw, rw)
    torch.cuda.synchronize()
    assert pair.gc.status == 0
    assert_same_cache(pair.oc, pair.gc.state_numpy())
    pair.append_step(9)
    assert_same_cache(pair.oc, pair.gc.state_numpy())
    ref, got = pair.decode(wl.queries(w, 3))
    assert_attention_close(ref, got)
    assert_mass_close(pair.oc.st["seq_len"], ref, got)


def test_running_sums_past_48_bits():
    """70,000 candidates scoring near the 2^16 clamp: the fixed-point running
    sum passes 2^48 (the packed word's field), which the budgets must not
    notice."""
    rng = np.random.default_rng(41)
    n = 70_000
    row = list(np.repeat(rng.integers(0, 3, n // 10), rng.integers(10, 40, n // 10)))[:n]
    log(f"[gpu tam] running sums past 2^48: {len(row)} tokens")
    oc, gc, g = _pair_from_tags([row])
    sc = np.zeros((1, g.n_cap), dtype=np.float32)
    sc[0, :n] = rng.uniform(60000.0, 65535.0, n).astype(np.float32)
    assert float(np.floor(sc.astype(np.float64) * 65536).sum()) > 2.0 ** 48
    _run_both(oc, gc, g, sc, 5000, INF, 1, 16, 32)
    assert_same_cache(oc, gc.state_numpy())
