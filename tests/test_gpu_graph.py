"""The decode loop captured in HIP graphs and replayed, against the same calls
made eagerly on a twin cache: one graph holds a step (append, then decode
with the decayed importance), another the windowed top-k prune ("ThinKV",
Continuous Thinking; "Dynamic Thinking-Token Selection ...", 2.3).  The
append and the eviction rank pops and pushes across workgroups with words
tagged by an epoch the device keeps, so replaying one captured launch must
behave as a fresh call each time.

Between replays the test runs its own eager work (the next step's inputs
copied into the graph's input tensors, a synchronisation, host copies), and
after every replay compares output, mass, importance and the whole cache
state bit for bit with the eager twin: both run the same kernels in the same
order on the same inputs."""
import numpy as np
import pytest

from eviction_kvq_decode_amd import workloads as wl
from pairs import log

pytestmark = pytest.mark.gpu
HD = 128


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_match_eager(noalloc):
    import torch

    from eviction_kvq_decode_amd import kvq

    w = wl.scaled(wl.WORKLOADS["ct_loop"], B=16, n_min=600, n_max=600, keep=300, q_window=32,
                  recent_window=64, period=16, loop_steps=64, extra_steps=64 + 16)
    log(f"[gpu graph] noalloc={noalloc} B={w.B} Hq={w.Hq} Hkv={w.Hkv} cached={w.n_min} "
        f"budget={w.keep} period={w.period} steps={w.loop_steps}")
    n0 = w.n_min
    toks = wl.lockstep_tokens(w, n0 + w.extra_steps)
    g = wl.geometry_for(w, toks.seq_tags)
    state = wl.empty_state(g, w.identity_ids, seed_key=(w.wid,))
    eager, graphed = kvq.Cache(g, state), kvq.Cache(g, state)
    K, V, T = (torch.from_numpy(a).cuda() for a in (toks.k, toks.v, toks.tags))
    for i in range(n0):
        eager.append(K[i], V[i], T[i])
        # (the no-allocation append looks its scratch up on first use: not
        # under capture)
        (graphed.append_noalloc if noalloc else graphed.append)(K[i], V[i], T[i])
    torch.cuda.synchronize()
    tags_all = wl.loop_tags(w, n0 + w.loop_steps)

    def fresh(shape, dtype, fill=0.0):
        return torch.full(shape, fill, dtype=dtype, device="cuda")

    io = {}
    for name, c in (("e", eager), ("g", graphed)):
        io[name] = dict(k=fresh((w.B, w.Hkv, HD), torch.float16), v=fresh((w.B, w.Hkv, HD), torch.float16),
                        t=fresh((w.B,), torch.uint8), q=fresh((w.B, w.Hq, HD), torch.float16),
                        out=fresh((w.B, w.Hq, HD), torch.float32), mass=fresh((w.B, g.n_cap), torch.float32),
                        imp=fresh((w.B, g.n_cap), torch.float32),
                        keep=torch.full((w.B,), w.keep, dtype=torch.int32, device="cuda"))

    def step(c, d):
        (c.append_noalloc if noalloc else c.append)(d["k"], d["v"], d["t"])
        c.decode(d["q"], d["out"], d["mass"], d["imp"], w.decay)

    def prune(c, d):
        c.evict(d["imp"], d["keep"], w.q_window, w.recent_window)

    gi = io["g"]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g_step, g_prune = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g_step, stream=side):
            step(graphed, gi)
        with torch.cuda.graph(g_prune, stream=side):
            prune(graphed, gi)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capturing ran nothing
    assert np.array_equal(eager.state_numpy()["seq_len"], graphed.state_numpy()["seq_len"])

    prunes = 0
    for s in range(w.loop_steps):
        k, v, tags = wl.loop_step_tokens(w, s, tags_all)
        q = wl.queries(w, s)
        for d in io.values():
            for key, a in (("k", k), ("v", v), ("t", tags), ("q", q)):
                d[key].copy_(torch.from_numpy(np.ascontiguousarray(a)))
        step(eager, io["e"])
        g_step.replay()
        pruned = (s + 1) % w.period == 0
        if pruned:
            prune(eager, io["e"])
            g_prune.replay()
            prunes += 1
        torch.cuda.synchronize()
        for key in ("out", "mass", "imp"):
            assert torch.equal(io["e"][key], gi[key]), f"step {s}: {key} differs"
        if pruned or s == w.loop_steps - 1:
            a, b = eager.state_numpy(), graphed.state_numpy()
            for key in a:
                assert np.array_equal(a[key], b[key]), f"step {s}: cache {key} differs"
    assert eager.status == 0 and graphed.status == 0
    assert prunes == w.loop_steps // w.period
