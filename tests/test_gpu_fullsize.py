"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the whole batch in one call).

The oracle computes a few sampled sequences (first, last, and for the ragged
batch the longest and shortest); every sequence of the batch is also checked
against properties that hold at any size.  Integer state of the sampled
sequences is compared bit for bit, output within 2e-3 relative / 1e-3
absolute, mass and importance within 1e-5 absolute.
"""
import numpy as np
import pytest

from eviction_kvq_decode_amd import workloads as wl
from fullsize import (FullPair, assert_pools_partitioned, assert_properties, assert_same_sequence,
                      assert_sample_close, valid_positions)
from pairs import log

pytestmark = pytest.mark.gpu


def _sample(w):
    n = wl.seq_lengths(w)
    return [0, w.B - 1, int(np.argmax(n)), int(np.argmin(n))]


def _check_sample_state(fp):
    gst, ost = fp.gc.state_numpy(), fp.oc.st
    for j, b in enumerate(fp.sample):
        assert_same_sequence(gst, fp.g, b, ost, fp.gs, j)
    return gst


def _decode_step(fp, step, importance=None, decay=0.0):
    q = wl.queries(fp.w, step)
    ref, got = fp.decode(q, importance, decay)
    gst = _check_sample_state(fp)
    assert_sample_close(ref, got, fp.sample, gst["seq_len"])
    assert_properties(gst, fp.g, got, fp.w.Hq)
    return gst, got


@pytest.mark.parametrize("name", ["llama8b", "long_evicted"])
def test_fullsize_decode(name):
    """Decode over the full Llama-8B-shaped batch, and the long evicted
    trace's timed step (append one token per sequence, then decode)."""
    w = wl.WORKLOADS[name]
    log(f"[gpu fullsize] {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.n_max}")
    fp = FullPair(w, _sample(w))
    fp.fill()
    _check_sample_state(fp)
    for step in range(w.append_steps):
        fp.append_step(step)
    assert fp.gc.status == 0
    _decode_step(fp, 0)
    del fp


def test_fullsize_decode_native_codec():
    """The long evicted trace's timed step with the cache in ThinKV's own
    formats (E4M3 / E2M1 / ternary), as `bench.py --codec native` times it."""
    w = wl.scaled(wl.WORKLOADS["long_evicted"], codec=1)
    log(f"[gpu fullsize] long_evicted, native codec: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.n_max}")
    fp = FullPair(w, _sample(w))
    fp.fill()
    _check_sample_state(fp)
    for step in range(w.append_steps):
        fp.append_step(step)
    assert fp.gc.status == 0
    _decode_step(fp, 0)
    del fp


@pytest.mark.parametrize("name", ["budgeted", "ragged"])
def test_fullsize_decode_importance_evict(name):
    """Decode with importance accumulation, then windowed top-k eviction with
    table compaction, over the whole batch."""
    w = wl.WORKLOADS[name]
    log(f"[gpu fullsize] {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N=[{w.n_min},{w.n_max}]")
    fp = FullPair(w, _sample(w))
    fp.fill()
    imp0 = np.stack([wl.importance0(w, b, fp.g.n_cap) for b in range(w.B)])
    gst, got = _decode_step(fp, 0, imp0, w.decay)
    imp_gpu = got[2]
    keep_k = wl.keep_counts(w)
    before = [valid_positions(gst, fp.g, b) for b in range(w.B)]
    fp.evict(imp_gpu, keep_k, w.q_window, w.recent_window)
    assert fp.gc.status == 0
    after_st = _check_sample_state(fp)
    # every sequence: windows kept, kept count = min(valid, k + windowed)
    for b in range(w.B):
        n = int(after_st["seq_len"][b])
        vb = before[b]
        win = (vb < w.q_window) | (vb >= n - w.recent_window)
        va = valid_positions(after_st, fp.g, b)
        assert np.all(np.isin(vb[win], va)), f"window evicted b={b}"
        assert va.size == min(vb.size, int(keep_k[b]) + int(win.sum())), f"kept count b={b}"
        # the kept non-window slots are the best by (importance desc, pos asc)
        cand = vb[~win]
        order = np.lexsort((cand, -imp_gpu[b, cand].astype(np.float64)))
        best = np.sort(cand[order[: int(keep_k[b])]])
        assert np.array_equal(np.sort(va[~np.isin(va, vb[win])]), best), f"top-k set b={b}"
    assert_pools_partitioned(after_st, fp.g)
    del fp


def test_fullsize_segment_eviction_and_budgets():
    """Thought-adaptive eviction by segment and thought-aware segment budgets
    over the whole budgeted batch (B=64, 16384 positions), from the same
    decoded state, with the parameters the benchmark times."""
    import bench

    w = wl.WORKLOADS["budgeted"]
    log(f"[gpu fullsize] segment eviction: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.n_max}")
    fp = FullPair(w, _sample(w))
    fp.fill()
    imp0 = np.stack([wl.importance0(w, b, fp.g.n_cap) for b in range(w.B)])
    gst, got = _decode_step(fp, 0, imp0, w.decay)
    imp_gpu = got[2]
    keep_k = wl.keep_counts(w)
    before = [valid_positions(gst, fp.g, b) for b in range(w.B)]
    snap = fp.snapshot()
    for policy in ("tbe", "tam"):
        log(f"[gpu fullsize] {policy}")
        fp.restore(snap)
        if policy == "tbe":
            fp.evict_tbe(imp_gpu, *bench.TBE_PARAMS, w.q_window, w.recent_window)
        else:
            fp.evict_tam(imp_gpu, keep_k, *bench.TAM_PARAMS, w.q_window, w.recent_window)
        assert fp.gc.status == 0
        after_st = _check_sample_state(fp)
        for b in range(w.B):
            n = int(after_st["seq_len"][b])
            vb = before[b]
            win = (vb < w.q_window) | (vb >= n - w.recent_window)
            va = valid_positions(after_st, fp.g, b)
            assert np.all(np.isin(vb[win], va)), f"{policy}: window evicted b={b}"
            assert np.all(np.isin(va, vb)), f"{policy}: a slot appeared b={b}"
            if policy == "tam":
                kept = int((~np.isin(va, vb[win])).sum())
                assert kept >= min(int(keep_k[b]), int((~win).sum())), f"tam: budget not used b={b}"
        assert_pools_partitioned(after_st, fp.g)
    del fp
