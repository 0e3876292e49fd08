"""GPU parity of the continuous-thinking loop (eviction_kvq_decode_amd.ct_loop)
against the oracle running the same loop: a generation under a cache budget,
pruned every P tokens ("ThinKV", Continuous Thinking; "TAM", section 2.D), by
windowed top-k, by thought segment (TBE) or by segment budgets (TAM).

Every step compares the output (2e-3 relative / 1e-3 absolute) and the mass
and importance (1e-5 absolute); after every prune the whole cache state is
compared bit for bit.  The oracle prunes with the GPU's importance, so that
importances equal to within rounding cannot pick different survivors; its
own importance is still compared at every step.
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
    tbe, tam = (16, 2, 4), (6.0, 8)
    ct = ContinuousThinking(gc, w.keep, w.period, w.q_window, w.recent_window, w.decay, policy=policy,
                            tbe=tbe, tam=tam)
    imp_o = np.zeros((w.B, g.n_cap), dtype=np.float32)
    keep = np.full(w.B, w.keep, dtype=np.int32)
    tags_all = wl.loop_tags(w, n0 + w.loop_steps)
    out = torch.empty((w.B, w.Hq, HD), device="cuda")
    mass = torch.full((w.B, g.n_cap), -7.0, device="cuda")
    prunes = 0
    for s in range(w.loop_steps):
        k, v, tags = wl.loop_step_tokens(w, s, tags_all)
        q = wl.queries(w, s)
        pruned = ct.step(*(torch.from_numpy(a).cuda() for a in (k, v, tags, q)), out, mass)
        oc.append(k, v, tags)
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
        if pruned:
            # the importance the GPU pruned with is the one after this decode
            imp_g = ct.importance.cpu().numpy()
            ei = np.abs(imp_g - imp_o)
            assert ei.max() <= ATOL_MASS, f"step {s} importance: {ei.max():.3g}"
            if policy == "tbe":
                oc.evict_tbe(imp_g, *tbe, w.q_window, w.recent_window)
            elif policy == "tam":
                oc.evict_tam(imp_g, keep, *tam, w.q_window, w.recent_window)
            else:
                oc.evict(imp_g, keep, w.q_window, w.recent_window)
            assert_same_cache(oc, gc.state_numpy())
            prunes += 1
    assert prunes == w.loop_steps // w.period
    # the final importance, compared at every valid position
    ei = np.abs(ct.importance.cpu().numpy() - imp_o)
    assert ei.max() <= ATOL_MASS
