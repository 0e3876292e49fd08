"""Pins of the oracle's thought-aware budgets (orc_evict_tam).

"Thought-Aware KV Cache Compaction ... (TAM)", section 2: segments of the
trajectory (A), budgets t_i proportional to sqrt(w_i) n_i with w_i the mean
window score of the segment (B), and pivotal tokens above c times the mean
score kept exactly with the rest of the budget shared among the others (C).
Compaction is read as keeping a subset of the cached tokens.  The expected
survivors below are worked out by hand from that rule; scores are chosen so
that every mean is exact in the 16-fractional-bit fixed point.
"""
import math

import numpy as np

from helpers import oracle_cache, small_geometry

R, E, T = 0, 1, 2
INF = float("inf")


def _build(tags, scores, B=1):
    n = len(tags)
    g = small_geometry(B, 8, 2, n_max=max(n, 1))
    oc = oracle_cache(g, identity_ids=True)
    rng = np.random.default_rng(11)
    for t in tags:
        k = rng.standard_normal((B, 2, 128)).astype(np.float16)
        v = rng.standard_normal((B, 2, 128)).astype(np.float16)
        oc.append(k, v, np.full(B, t, dtype=np.uint8))
    sc = np.zeros((B, g.n_cap), dtype=np.float32)
    sc[:, :n] = np.asarray(scores, dtype=np.float32)
    return oc, sc


def _kept(oc, b=0):
    return sorted(p for (_, _, _, p) in oc.valid_slots(b))


def test_sqrt_rule_two_segments():
    # R segment, mean 4 (sqrt 2); E segment, mean 1 (sqrt 1); sizes 8 and 8:
    # shares 2:1 of T = 6 -> 4 and 2.  Inside each, the highest scores, ties
    # to the lower position.
    tags = [R] * 8 + [E] * 8
    scores = [3, 5] * 4 + [0.5, 1.5] * 4
    oc, sc = _build(tags, scores)
    oc.evict_tam(sc, 6, INF, 1, 0, 0)
    assert _kept(oc) == [1, 3, 5, 7, 9, 11]
    assert oc.status == 0


def test_capped_share_is_shared_again():
    # A (2 tokens, mean 100 -> sqrt 10, weight 20), B and C (10 tokens each,
    # mean 1, weight 10): shares of 8 are 4, 2, 2; A's share reaches its size
    # and is capped at 2; the 6 left go 3 and 3 to B and C.
    tags = [R] * 2 + [E] * 10 + [T] * 10
    scores = [100, 100] + [0.5, 1.5] * 5 + [0.5, 1.5] * 5
    oc, sc = _build(tags, scores)
    oc.evict_tam(sc, 8, INF, 1, 0, 0)
    assert _kept(oc) == [0, 1, 3, 5, 7, 13, 15, 17]


def test_pivotal_tokens_kept_outside_the_budget():
    # mean score 2; c = 3 -> threshold 6: only position 9 (11) is pivotal.
    # keep 4 -> 3 for the others (all equal: the lowest positions).
    tags = [R] * 10
    scores = [1] * 9 + [11]
    oc, sc = _build(tags, scores)
    oc.evict_tam(sc, 4, 3.0, 1, 0, 0)
    assert _kept(oc) == [0, 1, 2, 9]
    # a budget below the pivotal count still keeps every pivotal token
    oc, sc = _build(tags, scores)
    oc.evict_tam(sc, 0, 3.0, 1, 0, 0)
    assert _kept(oc) == [9]


def test_weights_use_segment_mean_and_non_pivotal_count():
    # A: 8 tokens, seven at 1 and one at 57 (mean 8); B: 8 tokens at 8 (mean
    # 8).  Overall mean 8, c = 3 -> threshold 24: position 7 is pivotal.
    # keep 9 -> T = 8 for the 7 + 8 others.  Weights sqrt(8) * 7 and
    # sqrt(8) * 8: shares 3.73 and 4.27 -> running floors 3, 8 -> budgets 3
    # and 5.  (Weights by the full sizes would give 4 and 4; by the mean of
    # the non-pivotal tokens, 1 and 7.)
    tags = [R] * 8 + [E] * 8
    scores = [1] * 7 + [57] + [8] * 8
    oc, sc = _build(tags, scores)
    oc.evict_tam(sc, 9, 3.0, 1, 0, 0)
    assert _kept(oc) == [0, 1, 2, 7, 8, 9, 10, 11, 12]


def test_short_runs_merge_into_the_segment_before():
    # R R R E R R R E E E, scores 9 9 9 1 4 4 4 2 2 2, keep 5.
    # min_seg 2: the lone E (a run of 1) joins the first segment:
    # {0..3} (mean 7, sqrt 2.65, weight 10.6), {4,5,6} (mean 4, weight 6),
    # {7,8,9} (mean 2, weight 4.2): shares 2.55, 1.44, 1.01 -> running floors
    # 2, 3, 5 -> budgets 2, 1, 2: positions 0, 1 | 4 | 7, 8.
    # min_seg 1: {0,1,2} (mean 9, weight 9), {3} (mean 1, weight 1), {4,5,6}
    # (weight 6), {7,8,9} (weight 4.2): shares 2.23, 0.25, 1.49, 1.04 ->
    # running floors 2, 2, 3, 5 -> budgets 2, 0, 1, 2: the same positions.
    # min_seg 4: every run after the first is shorter than 4, so all of them
    # join the first segment: one segment keeps its best 5, the three 9s and
    # the first two 4s: positions 0, 1, 2, 4, 5.
    tags = [R, R, R, E, R, R, R, E, E, E]
    scores = [9, 9, 9, 1, 4, 4, 4, 2, 2, 2]
    for min_seg, expect in [(2, [0, 1, 4, 7, 8]), (1, [0, 1, 4, 7, 8]), (4, [0, 1, 2, 4, 5])]:
        oc, sc = _build(tags, scores)
        oc.evict_tam(sc, 5, INF, min_seg, 0, 0)
        assert _kept(oc) == expect, min_seg


def test_windows_and_degenerate_budgets():
    tags = [R] * 6 + [E] * 6
    scores = [float(i + 1) for i in range(12)]
    # windows: positions 0, 1 and 10, 11 stay and are not candidates
    oc, sc = _build(tags, scores)
    oc.evict_tam(sc, 0, INF, 1, 2, 2)
    assert _kept(oc) == [0, 1, 10, 11]
    # a budget of at least the candidates keeps everything
    oc, sc = _build(tags, scores)
    oc.evict_tam(sc, 100, INF, 1, 0, 0)
    assert _kept(oc) == list(range(12))
    # zero scores: every weight is 0 and only the windows stay
    oc, sc = _build(tags, [0.0] * 12)
    oc.evict_tam(sc, 5, INF, 1, 1, 1)
    assert _kept(oc) == [0, 11]
    # no candidates at all
    oc, sc = _build([], [])
    oc.evict_tam(sc, 5, 2.0, 1, 0, 0)
    assert oc.status == 0


def _real_budgets(sizes, means, T):
    """Real-valued water-filling of T over segments with weights
    sqrt(mean) * size, sizes as caps (written from the rule, in float64)."""
    w = [math.sqrt(m) * s for m, s in zip(means, sizes)]
    x = [None] * len(sizes)
    free = set(range(len(sizes)))
    left = float(T)
    while True:
        tot = sum(w[i] for i in free)
        over = [i for i in free if tot > 0 and left * w[i] / tot >= sizes[i]]
        if not over:
            for i in free:
                x[i] = left * w[i] / tot if tot > 0 else 0.0
            return x
        for i in over:
            x[i] = float(sizes[i])
            left -= sizes[i]
            free.discard(i)


def test_budgets_follow_the_real_rule_within_one():
    rng = np.random.default_rng(5)
    for trial in range(20):
        n_seg = int(rng.integers(2, 12))
        sizes = [int(x) for x in rng.integers(1, 30, n_seg)]
        tags = []
        for i, s in enumerate(sizes):
            tags += [(R, E, T)[i % 3]] * s
        # one score per segment, a multiple of 1/16 (exact mean in fixed point)
        seg_scores = [float(x) for x in np.round(rng.exponential(2.0, n_seg) * 16 + 1) / 16]
        scores = sum(([v] * s for v, s in zip(seg_scores, sizes)), [])
        keep = int(rng.integers(0, sum(sizes) + 1))
        oc, sc = _build(tags, scores)
        oc.evict_tam(sc, keep, INF, 1, 0, 0)
        kept = np.array(_kept(oc))
        starts = np.cumsum([0] + sizes)
        got = [int(((kept >= starts[i]) & (kept < starts[i + 1])).sum()) for i in range(n_seg)]
        want = _real_budgets(sizes, seg_scores, keep)
        assert sum(got) == keep
        for g_, w_, s in zip(got, want, sizes):
            assert g_ <= s and abs(g_ - w_) < 1 + 1e-9, (trial, got, want)
