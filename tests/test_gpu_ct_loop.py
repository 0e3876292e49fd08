"""GPU parity of the continuous-thinking loop (eviction_kvq_decode_amd.ct_loop)
against the oracle running the same loop: a generation under a cache budget
("ThinKV", Continuous Thinking), pruned
  - topk: every P tokens, windowed top-k on the decayed importance;
  - tbe: at every step where a Transition thought starts, in those sequences
    only ("ThinKV", think-before-evict), by thought segment;
  - tam: every P tokens ("TAM", 2.D) by segment budgets, on the mass the last
    R queries gave each position (the selection window, "TAM", 2.B).

Every step compares the output (2e-3 relative / 1e-3 absolute) and the mass
(1e-5 absolute); after every prune the whole cache state is compared bit for
bit.  The oracle prunes with the GPU's importance (or window score), so that
scores equal to within rounding cannot pick different survivors; the
importance is compared to 1e-5 and the window score to R x 1e-5.
"""
import math

import numpy as np
import pytest

from eviction_kvq_decode_amd import workloads as wl
from pairs import ATOL_MASS, assert_attention_close, assert_same_cache, log
from oracle import oracle as orc

pytestmark = pytest.mark.gpu
HD = 128


@pytest.mark.parametrize("policy", ["topk", "tbe", "tam"])
def test_ct_loop_matches_oracle(policy):
    import torch

    from eviction_kvq_decode_amd import kvq
    from eviction_kvq_decode_amd.ct_loop import ContinuousThinking

    w = wl.scaled(wl.WORKLOADS["ct_loop"], B=3, n_min=1200, n_max=1200, keep=500,
                  q_window=64, recent_window=128, period=64, loop_steps=320, extra_steps=320 + 16)
    log(f"[gpu ct loop] {policy}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} cached={w.n_min} budget={w.keep} "
        f"period={w.period} steps={w.loop_steps}")
    n0 = w.n_min
    toks = wl.lockstep_tokens(w, n0 + w.extra_steps)
    g = wl.geometry_for(w, toks.seq_tags)
    state = wl.empty_state(g, w.identity_ids, seed_key=(w.wid,))
    oc, gc = orc.OracleCache(g, state), kvq.Cache(g, state)
    K, V, T = (torch.from_numpy(a).cuda() for a in (toks.k, toks.v, toks.tags))
    for i in range(n0):
        oc.append(toks.k[i], toks.v[i], toks.tags[i])
        gc.append(K[i], V[i], T[i])
    torch.cuda.synchronize()
    tbe, tam = (16, 2, 4), (6.0, 8, 16)
    tags_all = wl.loop_tags(w, n0 + w.loop_steps)
    last_tags = tags_all[np.arange(w.B), n0 - 1]
    ct = ContinuousThinking(gc, w.keep, w.period, w.q_window, w.recent_window, w.decay, policy=policy,
                            tbe=tbe, tam=tam, last_tags=last_tags)
    imp_o = np.zeros((w.B, g.n_cap), dtype=np.float32)     # decayed importance (topk, tbe)
    win_o = np.zeros((w.B, g.n_cap), dtype=np.float32)     # window score (tam)
    keep = np.full(w.B, w.keep, dtype=np.int32)
    out = torch.empty((w.B, w.Hq, HD), device="cuda")
    mass = torch.full((w.B, g.n_cap), -7.0, device="cuda")
    prunes = fired = 0
    prev = last_tags.copy()
    since = 0
    for s in range(w.loop_steps):
        k, v, tags = wl.loop_step_tokens(w, s, tags_all)
        q = wl.queries(w, s)
        pruned = ct.step(*(torch.from_numpy(a).cuda() for a in (k, v, tags, q)), out, mass, tags_host=tags)
        # the same loop on the oracle
        oc.append(k, v, tags)
        since += 1
        if policy == "tam":
            first = w.period - tam[2] + 1
            if since >= first:
                out_o, mass_o, win_o = oc.decode(q, 1 / math.sqrt(HD), win_o, 0.0 if since == first else 1.0)
                win_o = win_o.astype(np.float32)
            else:
                out_o, mass_o, _ = oc.decode(q, 1 / math.sqrt(HD))
        else:
            out_o, mass_o, imp_o = oc.decode(q, 1 / math.sqrt(HD), imp_o, w.decay)
            imp_o = imp_o.astype(np.float32)
        torch.cuda.synchronize()
        assert gc.status == 0 and int(oc.st["status"][0]) == 0
        n = oc.st["seq_len"].astype(np.int64)
        got = (out.cpu().numpy(), mass.cpu().numpy(), None)
        assert_attention_close((out_o, mass_o, None), got)
        for b in range(w.B):
            e = np.abs(got[1][b, : n[b]] - mass_o[b, : n[b]])
            assert e.max() <= ATOL_MASS, f"step {s} mass b={b}: {e.max():.3g}"
        onset = ((tags == 2) & (prev != 2)).astype(np.uint8)
        prev = tags.copy()
        if policy == "tbe":
            # fires exactly where a Transition starts
            assert pruned == bool(onset.any())
            if pruned:
                imp_g = ct.importance.cpu().numpy()
                assert np.abs(imp_g - imp_o).max() <= ATOL_MASS
                oc.evict_tbe(imp_g, *tbe, w.q_window, w.recent_window, seq_mask=onset)
                assert_same_cache(oc, gc.state_numpy())
                fired += int(onset.sum())
            continue
        assert pruned == (since == w.period)
        if pruned:
            since = 0
            if policy == "tam":
                # the window score the GPU pruned with: the mass of the last R queries
                sc_g = ct.window_score.cpu().numpy()
                for b in range(w.B):
                    e = np.abs(sc_g[b, : n[b]] - win_o[b, : n[b]])
                    # only valid positions are scored (and read by the eviction)
                    valid = np.zeros(n[b], bool)
                    for (_, _, _, pp) in oc.valid_slots(b):
                        valid[pp] = True
                    assert e[valid].max() <= tam[2] * ATOL_MASS, f"step {s} window score"
                oc.evict_tam(sc_g, keep, *tam[:2], w.q_window, w.recent_window)
            else:
                imp_g = ct.importance.cpu().numpy()
                assert np.abs(imp_g - imp_o).max() <= ATOL_MASS, f"step {s} importance"
                oc.evict(imp_g, keep, w.q_window, w.recent_window)
            assert_same_cache(oc, gc.state_numpy())
            prunes += 1
    if policy == "tbe":
        assert fired > 0
        log(f"[gpu ct loop] tbe fired {fired} times over {w.B} sequences")
    else:
        assert prunes == w.loop_steps // w.period
    if policy != "tam":
        # the final importance, compared at every valid position
        assert np.abs(ct.importance.cpu().numpy() - imp_o).max() <= ATOL_MASS
