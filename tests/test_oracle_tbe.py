"""Pins of the oracle's thought-adaptive eviction (orc_evict_tbe).

"ThinKV", Methodology, think-before-evict: once a Transition thought starts,
earlier Reasoning / Execution segments are pruned at segment granularity on
an annealing schedule (retention r0, r0/2, r0/4, ... for each further
Transition), and a small safety net of earlier Transition segments stays.
The expected survivors below are worked out by hand from that rule.
"""
import numpy as np

from helpers import oracle_cache, small_geometry

R, E, T = 0, 1, 2


def _build(tags, imp_by_pos, B=1):
    n = len(tags)
    g = small_geometry(B, 8, 2, n_max=n)
    oc = oracle_cache(g, identity_ids=True)
    rng = np.random.default_rng(11)
    for i, t in enumerate(tags):
        k = rng.standard_normal((B, 2, 128)).astype(np.float16)
        v = rng.standard_normal((B, 2, 128)).astype(np.float16)
        oc.append(k, v, np.full(B, t, dtype=np.uint8))
    imp = np.zeros((B, g.n_cap), dtype=np.float32)
    for p, x in imp_by_pos.items():
        if p < g.n_cap:
            imp[:, p] = x
    return oc, imp


def _kept(oc, b=0):
    return sorted(p for (_, _, _, p) in oc.valid_slots(b))


# positions:      0  1  2  3  4  5  6  7  8  9 10 11 12 13 14 15 16
TAGS = [R, R, R, R, E, E, E, T, T, R, R, R, R, R, T, E, E]
IMP = {0: 0.1, 1: 0.5, 2: 0.3, 3: 0.5,          # segment A (R)
       4: 0.2, 5: 0.9, 6: 0.1,                  # B (E)
       7: 0.4, 8: 0.6,                          # C (T)
       9: 0.05, 10: 0.7, 11: 0.7, 12: 0.2, 13: 0.8,  # D (R)
       14: 0.3,                                 # E (T)
       15: 0.1, 16: 0.2}                        # F (E)


def test_hand_worked_schedule_no_windows():
    # r0 = 2, r_min = 1, t_keep = 1.  Later Transition segments: F 0, E 0,
    # D 1, C 1, B 2, A 2.  F and E keep all; D keeps 2 >> 0 = 2 (13, then
    # 10 over 11 at equal importance); C (T) keeps t_keep = 1 (8); B keeps
    # max(1, 2 >> 1) = 1 (5); A keeps 1 (1 over 3 at equal importance).
    oc, imp = _build(TAGS, IMP)
    oc.evict_tbe(imp, 2, 1, 1, 0, 0)
    assert _kept(oc) == [1, 5, 8, 10, 13, 14, 15, 16]
    assert oc.status == 0


def test_hand_worked_schedule_with_windows():
    # question window 2 (positions 0, 1), recent window 2 (15, 16): those
    # stay and do not form segments.  Candidates 2..14: A' = {2, 3} (R), B,
    # C, D, E as above.  A' keeps 1: 3 (0.5 over 0.3).
    oc, imp = _build(TAGS, IMP)
    oc.evict_tbe(imp, 2, 1, 1, 2, 2)
    assert _kept(oc) == [0, 1, 3, 5, 8, 10, 13, 14, 15, 16]


def test_floor_and_emptied_block_is_freed():
    # E E E T R R T with r0 = 1, r_min = 0, t_keep = 0: the E segment has two
    # later Transitions (keeps max(0, 1 >> 1) = 0), the first T segment one
    # (keeps t_keep = 0), the R segment one (keeps 1 >> 0 = 1: position 5),
    # the last T segment none (keeps all).  The E block empties: it leaves
    # the table and its id goes back on the E free stack.
    tags = [E, E, E, T, R, R, T]
    imp = {0: 0.9, 1: 0.8, 2: 0.7, 3: 0.5, 4: 0.1, 5: 0.2, 6: 0.3}
    oc, im = _build(tags, imp)
    row_before = oc.table_row(0)
    e_ids = [int(x & 0x3FFFFFFF) for x in row_before if x >> 30 == E]
    top_e = int(oc.st["free_top"][E])
    oc.evict_tbe(im, 1, 0, 0, 0, 0)
    assert _kept(oc) == [5, 6]
    row_after = oc.table_row(0)
    assert [int(x >> 30) for x in row_after] == [int(x >> 30) for x in row_before if x >> 30 != E]
    assert int(oc.st["free_top"][E]) == top_e + 1
    assert int(oc.st["free1"][top_e]) == e_ids[0]


def test_no_transition_keeps_everything():
    tags = [R] * 20 + [E] * 20 + [R] * 5
    imp = {p: float(p) for p in range(len(tags))}
    oc, im = _build(tags, imp)
    oc.evict_tbe(im, 1, 0, 0, 0, 0)
    assert _kept(oc) == list(range(len(tags)))


def test_generous_retention_keeps_everything():
    rng = np.random.default_rng(3)
    tags = list(rng.integers(0, 3, 200))
    imp = {p: float(x) for p, x in enumerate(rng.random(200))}
    oc, im = _build(tags, imp)
    oc.evict_tbe(im, 1 << 20, 1 << 20, 1 << 20, 0, 0)
    assert _kept(oc) == list(range(200))


def test_retention_never_grows_with_more_transitions():
    # the same prefix followed by more Transition segments never keeps more
    rng = np.random.default_rng(4)
    base = [R] * 40 + [E] * 30
    imp = {p: float(x) for p, x in enumerate(rng.random(200))}
    kept = []
    for n_t in range(1, 6):
        tags = base + sum(([T] * 3 + [E] * 2 for _ in range(n_t)), [])
        oc, im = _build(tags, imp)
        oc.evict_tbe(im, 16, 1, 1, 0, 0)
        kept.append(sum(1 for p in _kept(oc) if p < len(base)))
    assert kept == sorted(kept, reverse=True) and kept[-1] < kept[0]
    assert kept[0] == 16 + 16 and kept[1] == 8 + 8 and kept[2] == 4 + 4


def test_sequence_mask_fires_per_sequence():
    # "ThinKV", think-before-evict: eviction is triggered where a Transition
    # thought is detected, so it runs per sequence.  Two sequences with the
    # same tokens; only sequence 1 is in the mask.  Sequence 0 keeps every
    # slot, and also the block whose slots were all cleared before the call
    # (an unmasked call would drop it from the table); sequence 1 ends as
    # the hand-worked schedule.
    oc, imp = _build(TAGS, IMP, B=2)
    ent0 = int(oc.st["table"][0])
    pool, bid = ent0 >> 30, ent0 & 0x3FFFFFFF
    oc.st[f"mask{pool}"][bid] = 0          # sequence 0's first block, emptied by hand
    before = {k: v.copy() for k, v in oc.st.items()}
    kept0 = _kept(oc, 0)
    oc.evict_tbe(imp, 2, 1, 1, 0, 0, seq_mask=np.array([0, 1], dtype=np.uint8))
    assert _kept(oc, 0) == kept0
    g = oc.g
    row0 = slice(0, g.max_blocks)
    assert np.array_equal(oc.st["table"][row0], before["table"][row0])
    assert int(oc.st["n_blocks"][0]) == int(before["n_blocks"][0])
    assert _kept(oc, 1) == [1, 5, 8, 10, 13, 14, 15, 16]
    # a mask of ones is the unmasked call
    oc2, imp2 = _build(TAGS, IMP, B=2)
    oc3, _ = _build(TAGS, IMP, B=2)
    oc2.evict_tbe(imp2, 2, 1, 1, 0, 0, seq_mask=np.ones(2, dtype=np.uint8))
    oc3.evict_tbe(imp2, 2, 1, 1, 0, 0)
    for k in oc2.st:
        assert np.array_equal(oc2.st[k], oc3.st[k]), k
