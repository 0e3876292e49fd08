"""Pins of the continuous-thinking loop on the oracle: a long generation
under a cache budget, pruned every P new tokens.

"ThinKV", Methodology, System Implementation (Continuous Thinking): evicted
slots are reused in place by later tokens of the same thought type, so the
cache footprint stays bounded without any compaction of KV bytes.  "TAM",
section 2.D: pruning every P tokens keeps the cache between the budget t and
t + P.  "Dynamic Thinking-Token Selection", section 2.3: windows are kept.

The pools here hold fewer slots than the generation appends tokens:
finishing without a full-pool status, with most appends landing in slots
that held an evicted token, is the reuse pin.
"""
import math

import numpy as np

from eviction_kvq_decode_amd import workloads as wl
from helpers import oracle_cache

HD = 128
BLK = 16


def _slots(st, g, b):
    """{(pool, id, slot): position} of the slots of sequence b's table blocks,
    and the positions of its valid slots."""
    nb = int(st["n_blocks"][b])
    row = st["table"][b * g.max_blocks: b * g.max_blocks + nb]
    allp, valid = {}, []
    for ent in row:
        p, bid = int(ent >> 30), int(ent & 0x3FFFFFFF)
        m = int(st[f"mask{p}"][bid])
        for s in range(BLK):
            allp[(p, bid, s)] = int(st[f"pos{p}"][bid * BLK + s])
            if (m >> s) & 1:
                valid.append(int(st[f"pos{p}"][bid * BLK + s]))
    return allp, np.asarray(valid, dtype=np.int64)


def test_loop_keeps_budget_windows_and_reuses_slots():
    w = wl.scaled(wl.WORKLOADS["ct_loop"], B=2, Hq=8, Hkv=2, n_min=0, n_max=0,
                  keep=96, q_window=16, recent_window=32, period=32, loop_steps=1024)
    budget, P, qw, rw = w.keep, w.period, w.q_window, w.recent_window
    n_total = w.loop_steps
    # room for the live set (budget + windows + P, plus a partly filled block
    # per type) in each pool, far less than the tokens appended in total
    per_pool = w.B * (math.ceil((budget + qw + rw + P) / BLK) + 4)
    g = wl.Geometry(w.B, w.Hq, w.Hkv, max_blocks=3 * per_pool // w.B, n_cap=n_total + 16,
                    pool_blocks=(per_pool, per_pool, per_pool))
    assert 3 * per_pool * BLK < w.B * n_total
    oc = oracle_cache(g, seed_key=(w.wid,))
    tags_all = wl.loop_tags(w, n_total)
    rng = np.random.default_rng(5)
    imp = np.zeros((w.B, g.n_cap), dtype=np.float32)
    reused = prunes = 0
    for i in range(n_total):
        k = rng.standard_normal((w.B, w.Hkv, HD)).astype(np.float16)
        v = rng.standard_normal((w.B, w.Hkv, HD)).astype(np.float16)
        pos_before = [oc.st[f"pos{p}"].copy() for p in range(3)]
        oc.append(k, v, np.ascontiguousarray(tags_all[:, i]))
        assert int(oc.st["status"][0]) == 0, f"pool or table full at token {i}"
        for b in range(w.B):
            new = [s for s, pos in _slots(oc.st, g, b)[0].items() if pos == i]
            assert len(new) == 1, f"token {i} of sequence {b} not placed once"
            # the slot held an earlier token: reused in place, or in a block
            # that was freed and popped again (its slots keep old positions)
            p, bid, sl = new[0]
            reused += int(pos_before[p][bid * BLK + sl]) != -1
        q = rng.standard_normal((w.B, w.Hq, HD)).astype(np.float16)
        _, _, imp = oc.decode(q, 1 / math.sqrt(HD), imp, w.decay)
        imp = imp.astype(np.float32)
        if (i + 1) % P == 0:
            prunes += 1
            n_now = oc.st["seq_len"].astype(np.int64)
            pre = [_slots(oc.st, g, b)[1] for b in range(w.B)]
            oc.evict(imp, np.full(w.B, budget, dtype=np.int32), qw, rw)
            for b in range(w.B):
                post = _slots(oc.st, g, b)[1]
                win = (pre[b] < qw) | (pre[b] >= n_now[b] - rw)
                assert np.all(np.isin(pre[b][win], post)), "a windowed token was evicted"
                outside = post[~np.isin(post, pre[b][win])]
                assert outside.size == min(budget, int((~win).sum()))
                assert post.size <= budget + qw + rw
    assert prunes == n_total // P
    # once the budget is reached, nearly every append lands in a used slot
    assert reused > w.B * (n_total - 2 * (budget + qw + rw + P))

