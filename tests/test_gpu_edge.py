"""GPU edge cases against the oracle: empty and skipped sequences, pool
exhaustion, bad tags, GQA group sizes 1 and 16, empty blocks left in the
table, degenerate eviction budgets, and the closed forms of attention."""
import math

import numpy as np
import pytest

from eviction_kvq_decode_amd import workloads as wl
from helpers import small_geometry
from oracle import oracle as orc
from pairs import assert_attention_close, assert_mass_close, assert_same_cache, log

pytestmark = pytest.mark.gpu

HD = 128
SM = 1 / math.sqrt(HD)


def _mk(g, identity=True, state=None):
    from eviction_kvq_decode_amd import kvq

    st = wl.empty_state(g, identity) if state is None else state
    return orc.OracleCache(g, st), kvq.Cache(g, st)


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _append(oc, gc, k, v, tags):
    oc.append(k, v, tags)
    gc.append(_dev(k), _dev(v), _dev(np.asarray(tags, np.uint8)))


def _decode(oc, gc, q, imp=None, decay=0.0):
    import torch

    g = oc.g
    ref = oc.decode(q, SM, imp, decay)
    out = torch.full((g.B, g.Hq, HD), float("nan"), device="cuda")
    mass = torch.full((g.B, g.n_cap), -7.0, device="cuda")
    imp_d = None if imp is None else _dev(imp.astype(np.float32))
    gc.decode(_dev(q), out, mass, imp_d, decay)
    torch.cuda.synchronize()
    return ref, (out.cpu().numpy(), mass.cpu().numpy(), None if imp_d is None else imp_d.cpu().numpy())


def _fill(oc, gc, rng, n, tags_fn=None, kscale=1.0):
    g = oc.g
    for i in range(n):
        k = (rng.standard_normal((g.B, g.Hkv, HD)) * kscale).astype(np.float16)
        v = rng.standard_normal((g.B, g.Hkv, HD)).astype(np.float16)
        tags = rng.integers(0, 3, g.B).astype(np.uint8) if tags_fn is None else tags_fn(i)
        _append(oc, gc, k, v, tags)


def test_empty_and_skipped_sequences():
    log("[edge] empty and skipped sequences")
    g = small_geometry(3, 8, 2, 120)
    oc, gc = _mk(g)
    rng = np.random.default_rng(0)
    _fill(oc, gc, rng, 100, lambda i: np.array([i % 3, 255, (i // 7) % 3], np.uint8))
    assert_same_cache(oc, gc.state_numpy())
    q = rng.standard_normal((3, 8, HD)).astype(np.float16)
    ref, got = _decode(oc, gc, q)
    assert np.all(got[0][1] == 0.0)
    assert_attention_close(ref, got)
    assert_mass_close(oc.st["seq_len"], ref, got)


def test_pool_exhaustion_and_bad_tag():
    log("[edge] ENOSPC / EINVAL")
    g = wl.Geometry(3, 2, 1, 2, 64, (1, 1, 1))
    oc, gc = _mk(g)
    rng = np.random.default_rng(1)
    k = rng.standard_normal((3, 1, HD)).astype(np.float16)
    _append(oc, gc, k, k, np.array([0, 0, 2], np.uint8))
    assert oc.status == gc.status == -4
    assert_same_cache(oc, gc.state_numpy())
    oc.st["status"][0] = 0
    oc2, gc2 = _mk(g, state=oc.st)
    _append(oc2, gc2, k, k, np.array([7, 255, 255], np.uint8))
    assert oc2.status == gc2.status == -1
    assert_same_cache(oc2, gc2.state_numpy())
    # table full: max_blocks 2 and a third type
    oc3, gc3 = _mk(wl.Geometry(1, 2, 1, 2, 64, (4, 4, 4)))
    for tag in (0, 1, 2):
        _append(oc3, gc3, k[:1], k[:1], np.array([tag], np.uint8))
    assert oc3.status == gc3.status == -4
    assert_same_cache(oc3, gc3.state_numpy())


@pytest.mark.parametrize("codec", [0, 1], ids=["int", "native"])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (16, 1), (24, 2), (6, 2)])
def test_gqa_group_sizes(Hq, Hkv, codec):
    log(f"[edge] Hq={Hq} Hkv={Hkv} codec={codec}")
    g = small_geometry(2, Hq, Hkv, 700, codec=codec)
    oc, gc = _mk(g, identity=False)
    rng = np.random.default_rng(Hq)
    _fill(oc, gc, rng, 700)
    assert_same_cache(oc, gc.state_numpy())
    q = rng.standard_normal((2, Hq, HD)).astype(np.float16)
    imp = rng.exponential(0.1, (2, g.n_cap)).astype(np.float32)
    ref, got = _decode(oc, gc, q, imp, 0.9)
    assert_attention_close(ref, got)
    assert_mass_close(oc.st["seq_len"], ref, got)


def test_empty_blocks_left_in_table():
    log("[edge] empty blocks in table")
    g = small_geometry(2, 8, 2, 600)
    oc, gc = _mk(g, identity=False)
    rng = np.random.default_rng(3)
    _fill(oc, gc, rng, 600)
    st = gc.state_numpy()
    for b in range(2):
        for e in oc.table_row(b)[1::3]:
            p, bid = int(e >> 30), int(e & 0x3FFFFFFF)
            oc.st[f"mask{p}"][bid] = 0
            st[f"mask{p}"][bid] = 0
        for e in oc.table_row(b)[2::5]:
            p, bid = int(e >> 30), int(e & 0x3FFFFFFF)
            oc.st[f"mask{p}"][bid] &= 0x5A5A
            st[f"mask{p}"][bid] &= 0x5A5A
    _, gc2 = _mk(g, state=st)
    q = rng.standard_normal((2, 8, HD)).astype(np.float16)
    ref, got = _decode(oc, gc2, q)
    assert_attention_close(ref, got)
    assert_mass_close(oc.st["seq_len"], ref, got)


@pytest.mark.parametrize("B,n", [(1, 1000), (2, 1040), (40, 300)])
def test_full_tables_and_short_runs(B, n):
    """Tables filled to max_blocks (Reasoning tokens only, 16 to a block).
    A small batch is cut into short runs to spread over the workgroups, and
    a full table caps a sequence's run count at the partials it holds."""
    log(f"[edge] full tables B={B} n={n}")
    nbk = math.ceil(n / 16)
    g = small_geometry(B, 8, 2, n, max_blocks=nbk, n_cap=n + 16)
    oc, gc = _mk(g, identity=False)
    rng = np.random.default_rng(n)
    _fill(oc, gc, rng, n, lambda i: np.zeros(B, np.uint8))
    assert (gc.state_numpy()["n_blocks"] == nbk).all()
    q = rng.standard_normal((B, 8, HD)).astype(np.float16)
    imp = rng.exponential(0.1, (B, g.n_cap)).astype(np.float32)
    ref, got = _decode(oc, gc, q, imp, 0.9)
    assert_attention_close(ref, got)
    assert_mass_close(oc.st["seq_len"], ref, got)


@pytest.mark.parametrize("keep,qw,rw", [(0, 0, 0), (0, 10, 10), (10 ** 6, 0, 0), (5, 400, 400), (1, 0, 1)])
def test_degenerate_eviction(keep, qw, rw):
    log(f"[edge] evict keep={keep} qw={qw} rw={rw}")
    g = small_geometry(3, 4, 1, 300)
    oc, gc = _mk(g, identity=False)
    rng = np.random.default_rng(4)
    _fill(oc, gc, rng, 300)
    imp = rng.random((3, g.n_cap)).astype(np.float32)
    imp[1] = 0.5                                      # all ties
    kk = np.full(3, keep, np.int32)
    oc.evict(imp, kk, qw, rw)
    gc.evict(_dev(imp), _dev(kk), qw, rw)
    assert_same_cache(oc, gc.state_numpy())
    q = rng.standard_normal((3, 4, HD)).astype(np.float16)
    ref, got = _decode(oc, gc, q)
    assert_attention_close(ref, got)
    assert_mass_close(oc.st["seq_len"], ref, got)


def test_identical_keys_closed_form():
    log("[edge] identical keys")
    g = small_geometry(1, 8, 2, 300)
    oc, gc = _mk(g)
    rng = np.random.default_rng(5)
    kvec = rng.standard_normal((1, 2, HD)).astype(np.float16)
    vin = []
    for i in range(300):
        v = rng.standard_normal((1, 2, HD)).astype(np.float16)
        vin.append(v[0])
        _append(oc, gc, kvec, v, np.array([1], np.uint8))
    q = rng.standard_normal((1, 8, HD)).astype(np.float16)
    ref, got = _decode(oc, gc, q)
    assert np.all(np.abs(got[1][0, :300] - 8 / 300) <= 1e-5)
    vmean = np.stack([np.mean([oc.dequant_slot(p, b, kh, s)[1] for p, b, s, _ in oc.valid_slots(0)], axis=0)
                      for kh in range(2)])
    # the mean of the fp16 inputs themselves, within half a 4-bit step per
    # group (bounded from the inputs) plus the output tolerance
    vin = np.stack(vin).astype(np.float64).reshape(300, 2, 4, 32)
    half = (vin.max(axis=3) - vin.min(axis=3)) / 15 * (1 + 2.0 ** -10) * (0.5 + 2.0 ** -18)
    in_bound = np.repeat(half.mean(axis=0), 32, axis=1)          # [kv head][128]
    in_mean = vin.reshape(300, 2, HD).mean(axis=0)
    for h in range(8):
        assert np.all(np.abs(got[0][0, h] - vmean[h // 4]) <= 1e-3 + 2e-3 * np.abs(vmean[h // 4]))
        assert np.all(np.abs(got[0][0, h] - in_mean[h // 4]) <= in_bound[h // 4] + 1e-3 + 2e-3 * np.abs(in_mean[h // 4]))


def test_dominant_key_closed_form():
    log("[edge] dominant key")
    g = small_geometry(1, 4, 1, 200)
    oc, gc = _mk(g)
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 4, HD)).astype(np.float16)
    qm = q[0].astype(np.float32).mean(axis=0)
    for i in range(200):
        k = rng.standard_normal((1, 1, HD)).astype(np.float16)
        tag = rng.integers(0, 3)
        if i == 77:
            k[0, 0] = (40.0 * qm / np.abs(qm).max()).astype(np.float16)
            tag = 0
        _append(oc, gc, k, rng.standard_normal((1, 1, HD)).astype(np.float16), np.array([tag], np.uint8))
    ref, got = _decode(oc, gc, q)
    assert abs(got[1][0, 77] - 4.0) <= 1e-5
    vj = [oc.dequant_slot(p, b, 0, s)[1] for p, b, s, ps in oc.valid_slots(0) if ps == 77][0]
    for h in range(4):
        assert np.all(np.abs(got[0][0, h] - vj) <= 1e-3 + 2e-3 * np.abs(vj))


def test_append_first_free_slot_past_a_scan_round():
    """Long tables whose first free slot of the token's type lies past the
    first 1024 table entries (one scan round of the slot search) and past
    2048 (two rounds): the append must still take the first free slot in
    table order, and then the next ones, bit-exact with the oracle."""
    log("[edge] append: first free slot past a scan round")
    B, nent = 3, 2300
    g = small_geometry(B, 4, 1, 16 * nent, max_blocks=nent + 8, n_cap=16 * nent + 64,
                       pool_blocks=(B * nent, B * nent, B * nent))
    st = wl.empty_state(g, identity_ids=True)
    rng = np.random.default_rng(11)
    nxt = [0, 0, 0]
    # sequence b: full blocks of every type, and E blocks with one free slot
    # at these table entries (all later than the first scan round for b > 0)
    free_at = {0: [1100, 1500], 1: [2100, 2200], 2: [700, 1030]}
    for b in range(B):
        pos = 0
        for e in range(nent):
            p = 1 if e in free_at[b] else int(rng.integers(0, 3))
            if p == 1 and e not in free_at[b] and e % 7 == 0:
                p = 0
            bid = nxt[p]
            nxt[p] += 1
            st["table"][b * g.max_blocks + e] = (p << 30) | bid
            m = 0xFFFF
            if e in free_at[b]:
                m &= ~(1 << int(rng.integers(0, 16))) & 0xFFFF
            st[f"mask{p}"][bid] = m
            for s in range(16):
                if (m >> s) & 1:
                    st[f"pos{p}"][bid * 16 + s] = pos
                    pos += 1
        st["n_blocks"][b] = nent
        st["seq_len"][b] = pos
    for p in range(3):
        # pops hand out the ids above the ones in use
        free = np.zeros(g.pool_blocks[p], dtype=np.uint32)
        free[: g.pool_blocks[p] - nxt[p]] = np.arange(g.pool_blocks[p] - 1, nxt[p] - 1, -1)
        st[f"free{p}"] = free
        st["free_top"][p] = g.pool_blocks[p] - nxt[p]
    oc, gc = _mk(g, state=st)
    for i in range(4):
        k = rng.standard_normal((B, 1, HD)).astype(np.float16)
        v = rng.standard_normal((B, 1, HD)).astype(np.float16)
        _append(oc, gc, k, v, np.ones(B, np.uint8))
        gst = gc.state_numpy()
        assert_same_cache(oc, gst)
    # the first two appends filled the two holes of every sequence in order
    for b in range(B):
        for e in free_at[b]:
            ent = int(oc.table_row(b)[e])
            assert ent >> 30 == 1 and oc.st["mask1"][ent & 0x3FFFFFFF] == 0xFFFF


def test_maximum_batch_many_short_sequences():
    """The largest batch the library takes (B = 1024) of short sequences,
    some empty: each split workgroup's range crosses many (sequence, pack)
    units, and the finalize's sequence and item prefixes run to their last
    slot.  Decode with importance, then a top-k evict ranked across all
    1024 sequences, then decode again over the holes."""
    log("[edge] B=1024 short sequences")
    B, n = 1024, 48
    g = small_geometry(B, 32, 8, n)
    oc, gc = _mk(g, identity=False)
    rng = np.random.default_rng(1024)
    lens = rng.integers(0, n + 1, B)
    lens[rng.choice(B, 40, replace=False)] = 0
    tags_all = rng.integers(0, 3, (n, B)).astype(np.uint8)
    tags_all[np.arange(n)[:, None] >= lens[None, :]] = 255
    _fill(oc, gc, rng, n, lambda i: tags_all[i])
    assert_same_cache(oc, gc.state_numpy())
    assert (gc.state_numpy()["seq_len"] == lens).all()
    q = rng.standard_normal((B, 32, HD)).astype(np.float16)
    imp = rng.exponential(0.1, (B, g.n_cap)).astype(np.float32)
    ref, got = _decode(oc, gc, q, imp, 0.9)
    assert np.all(got[0][lens == 0] == 0.0)
    assert_attention_close(ref, got)
    assert_mass_close(oc.st["seq_len"], ref, got)
    # evict with the GPU's importance on both sides, so no near-tie differs
    imp_gpu = got[2]
    kk = rng.integers(0, 20, B).astype(np.int32)
    oc.evict(imp_gpu, kk, 2, 4)
    gc.evict(_dev(imp_gpu), _dev(kk), 2, 4)
    assert_same_cache(oc, gc.state_numpy())
    q2 = rng.standard_normal((B, 32, HD)).astype(np.float16)
    ref2, got2 = _decode(oc, gc, q2)
    assert_attention_close(ref2, got2)
    assert_mass_close(oc.st["seq_len"], ref2, got2)


def test_one_long_sequence_many_ranges():
    """One 16384-position sequence with 60% of its slots evicted (B=1, Hq=32,
    Hkv=8: two kv-head packs of about 490 table entries after the blocks the
    eviction emptied are freed).  The list is short against the split grid,
    so it goes to at most one workgroup per compute unit in ranges of at
    least 4 entries, about 125 ranges per pack, and the finalize merges each
    head's partials over 4 rounds of loads, in the head statistics and in the
    output rows.  Output, mass and importance against the oracle, then again
    after an append into the holes."""
    from pairs import Pair

    log("[edge] one long sequence, many split ranges")
    w = wl.scaled(wl.WORKLOADS["long_evicted"], B=1, n_min=16384, n_max=16384)
    p = Pair(w)
    p.fill()
    assert_same_cache(p.oc, p.gc.state_numpy())
    rng = np.random.default_rng(16384)
    imp = rng.exponential(1.0, size=(1, p.g.n_cap)).astype(np.float32)
    ref, got = p.decode(wl.queries(w, 0), imp, 0.9)
    assert_attention_close(ref, got)
    assert_mass_close(p.oc.st["seq_len"], ref, got)
    assert abs(got[1][0, : p.oc.st["seq_len"][0]].sum() - w.Hq) < 1e-3
    p.append_step(0)
    ref, got = p.decode(wl.queries(w, 1))
    assert_attention_close(ref, got)
    assert_mass_close(p.oc.st["seq_len"], ref, got)
