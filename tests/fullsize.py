"""Full-size workloads on the GPU, checked on sampled sequences against the
oracle and, for every sequence, against properties that hold at any size.

The GPU cache holds the whole batch.  The oracle holds only the sampled
sequences (an oracle cache of its own, so physical block ids differ); the
comparison of integer state is therefore made per sequence and independent
of ids: table order of pools, masks, positions and the bytes of every valid
slot.
"""
from __future__ import annotations

import math
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from eviction_kvq_decode_amd import workloads as wl
from oracle import oracle as orc
from pairs import ATOL_MASS, ATOL_OUT, RTOL_OUT, log, slot_byte_masks

HD = 128
BLK = 16
CHUNK = 2048          # positions per host->device chunk of the lock-step fill


class SeqTokens:
    """One sequence's cached tokens: tags, K, V and planned survivors."""

    def __init__(self, w: wl.Workload, b: int, n: int, n_cap: int):
        self.n = n
        self.tags, run = wl.tag_runs(w, b, n)
        self.k, self.v = wl.token_kv(w, b, n)
        self.keep = np.zeros(n_cap, dtype=bool)
        self.keep[:n] = wl.keep_plan(w, b, self.tags, run)


def lockstep_chunk(seqs: list, i0: int, i1: int, Hkv: int):
    """Position-major arrays [i1-i0][len(seqs)][...] for positions i0..i1-1."""
    B = len(seqs)
    k = np.zeros((i1 - i0, B, Hkv, HD), dtype=np.float16)
    v = np.zeros_like(k)
    t = np.full((i1 - i0, B), wl.TAG_SKIP, dtype=np.uint8)
    for j, s in enumerate(seqs):
        a, e = i0, min(i1, s.n)
        if e > a:
            k[: e - a, j] = s.k[a:e]
            v[: e - a, j] = s.v[a:e]
            t[: e - a, j] = s.tags[a:e]
    return k, v, t


def subset_geometry(g: wl.Geometry, seqs: list, w: wl.Workload) -> wl.Geometry:
    counts = np.zeros(3, dtype=np.int64)
    for s in seqs:
        for p in range(3):
            counts[p] += int(math.ceil(int((s.tags == p).sum()) / BLK))
    spare = len(seqs) * (4 + int(math.ceil((w.extra_steps + w.append_steps) / BLK)))
    return wl.Geometry(len(seqs), g.Hq, g.Hkv, g.max_blocks, g.n_cap,
                       tuple(int(c + spare) for c in counts), g.codec)


class FullPair:
    """The whole workload on the GPU; the sampled sequences on the oracle."""

    def __init__(self, w: wl.Workload, sample: list):
        import torch

        from eviction_kvq_decode_amd import kvq

        self.torch, self.w = torch, w
        n = wl.seq_lengths(w)
        self.n = n
        t0 = time.time()
        n_cap = int(n.max()) + w.extra_steps + w.append_steps
        with ThreadPoolExecutor(max_workers=16) as ex:
            self.seqs = list(ex.map(lambda b: SeqTokens(w, b, int(n[b]), n_cap), range(w.B)))
        self.g = wl.geometry_for(w, [s.tags for s in self.seqs])
        assert self.g.n_cap == n_cap
        self.sample = sorted(set(sample))
        log(f"  [{w.name}] tokens for B={w.B} (N up to {int(n.max())}) in {time.time() - t0:.1f}s")
        self.gc = kvq.Cache(self.g, wl.empty_state(self.g, w.identity_ids, seed_key=(w.wid,)))
        sub = [self.seqs[b] for b in self.sample]
        self.gs = subset_geometry(self.g, sub, w)
        self.oc = orc.OracleCache(self.gs, wl.empty_state(self.gs, w.identity_ids, seed_key=(w.wid, 1)))

    def fill(self):
        torch, w = self.torch, self.w
        t0 = time.time()
        n_max = int(self.n.max())
        sub = [self.seqs[b] for b in self.sample]
        for i0 in range(0, n_max, CHUNK):
            i1 = min(n_max, i0 + CHUNK)
            k, v, t = lockstep_chunk(self.seqs, i0, i1, w.Hkv)
            K, V, T = (torch.from_numpy(a).cuda() for a in (k, v, t))
            sk, sv, st = K[0].numel() * 2, V[0].numel() * 2, T[0].numel()
            kp, vp, tp = K.data_ptr(), V.data_ptr(), T.data_ptr()
            for i in range(i1 - i0):
                self.gc.append(kp + i * sk, vp + i * sv, tp + i * st)
            ko, vo, to = lockstep_chunk(sub, i0, i1, w.Hkv)
            for i in range(i1 - i0):
                self.oc.append(ko[i], vo[i], to[i])
            torch.cuda.synchronize()
            del K, V, T
        if w.holes > 0:
            keep = np.stack([s.keep for s in self.seqs])
            self.evict(keep.astype(np.float32), keep.sum(axis=1).astype(np.int32), 0, 0)
        assert self.gc.status == 0 and self.oc.status == 0
        log(f"  [{w.name}] filled in {time.time() - t0:.1f}s")

    def evict(self, imp_full, keep_full, qw, rw):
        """Evict on both sides with the same importance rows."""
        torch = self.torch
        self.gc.evict(torch.from_numpy(np.ascontiguousarray(imp_full, dtype=np.float32)).cuda(),
                      torch.from_numpy(np.ascontiguousarray(keep_full, dtype=np.int32)).cuda(), qw, rw)
        self.oc.evict(np.ascontiguousarray(imp_full[self.sample], dtype=np.float32),
                      np.ascontiguousarray(keep_full[self.sample], dtype=np.int32), qw, rw)

    def evict_tbe(self, imp_full, r0, r_min, t_keep, qw, rw):
        """Thought-adaptive eviction by segment on both sides."""
        torch = self.torch
        self.gc.evict_tbe(torch.from_numpy(np.ascontiguousarray(imp_full, dtype=np.float32)).cuda(),
                          r0, r_min, t_keep, qw, rw)
        self.oc.evict_tbe(np.ascontiguousarray(imp_full[self.sample], dtype=np.float32), r0, r_min, t_keep,
                          qw, rw)

    def evict_tam(self, score_full, keep_full, pivot_c, min_seg, qw, rw):
        """Thought-aware segment budgets on both sides."""
        torch = self.torch
        self.gc.evict_tam(torch.from_numpy(np.ascontiguousarray(score_full, dtype=np.float32)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(keep_full, dtype=np.int32)).cuda(),
                          pivot_c, min_seg, qw, rw)
        self.oc.evict_tam(np.ascontiguousarray(score_full[self.sample], dtype=np.float32),
                          np.ascontiguousarray(keep_full[self.sample], dtype=np.int32), pivot_c, min_seg, qw, rw)

    def snapshot(self):
        """Cache metadata of both sides (the KV bytes never change in eviction)."""
        return ({k: v.clone() for k, v in self.gc.t.items() if not k.startswith("kv")},
                {k: v.copy() for k, v in self.oc.st.items()})

    def restore(self, snap):
        gmeta, ost = snap
        for k, v in gmeta.items():
            self.gc.t[k].copy_(v)
        self.oc.st = {k: v.copy() for k, v in ost.items()}

    def append_step(self, step):
        torch = self.torch
        k, v, tags = wl.step_tokens(self.w, step)
        self.gc.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(tags).cuda())
        self.oc.append(k[self.sample], v[self.sample], tags[self.sample])

    def decode(self, q, importance=None, decay=0.0):
        """GPU decode of the whole batch; oracle decode of the sample."""
        torch, g = self.torch, self.g
        out = torch.full((g.B, g.Hq, HD), float("nan"), device="cuda")
        mass = torch.full((g.B, g.n_cap), -7.0, device="cuda")
        imp_dev = None
        if importance is not None:
            imp_dev = torch.from_numpy(np.ascontiguousarray(importance, dtype=np.float32)).cuda()
        self.gc.decode(torch.from_numpy(q).cuda(), out, mass, imp_dev, decay)
        torch.cuda.synchronize()
        got = (out.cpu().numpy(), mass.cpu().numpy(), None if imp_dev is None else imp_dev.cpu().numpy())
        imp_sub = None if importance is None else np.ascontiguousarray(importance[self.sample])
        ref = self.oc.decode(np.ascontiguousarray(q[self.sample]), 1 / math.sqrt(HD), imp_sub, decay)
        return ref, got


# ---------------------------------------------------------------- compare

_MASKS = {}


def _slot_masks(bits):
    if bits not in _MASKS:
        _MASKS[bits] = slot_byte_masks(bits)
    return _MASKS[bits]


def seq_layout(st: dict, g: wl.Geometry, b: int):
    """Per table entry of sequence b: (pool, id, mask, positions of valid slots)."""
    nb = int(st["n_blocks"][b])
    row = st["table"][b * g.max_blocks: b * g.max_blocks + nb]
    out = []
    for ent in row:
        p, bid = int(ent >> 30), int(ent & 0x3FFFFFFF)
        m = int(st[f"mask{p}"][bid])
        pos = st[f"pos{p}"][bid * BLK:(bid + 1) * BLK]
        out.append((p, bid, m, tuple(int(pos[s]) for s in range(BLK) if (m >> s) & 1)))
    return out


def assert_same_sequence(gst: dict, g: wl.Geometry, b: int, ost: dict, og: wl.Geometry, ob: int):
    """Bit-exact, id-independent comparison of one sequence's cache."""
    assert int(gst["seq_len"][b]) == int(ost["seq_len"][ob]), f"seq_len b={b}"
    A, Bo = seq_layout(gst, g, b), seq_layout(ost, og, ob)
    assert len(A) == len(Bo), f"n_blocks b={b}: gpu {len(A)} oracle {len(Bo)}"
    for e, (x, y) in enumerate(zip(A, Bo)):
        assert (x[0], x[2], x[3]) == (y[0], y[2], y[3]), f"b={b} table entry {e}: gpu {x} oracle {y}"
        p = x[0]
        bits = wl.POOL_BITS[p]
        rb = wl.region_bytes(bits)
        if x[2] == 0:
            continue
        sm = _slot_masks(bits)
        bm = np.zeros(rb, dtype=np.uint8)
        for s in range(BLK):
            if (x[2] >> s) & 1:
                bm |= sm[s]
        ra = gst[f"kv{p}"][x[1] * g.Hkv * rb:(x[1] + 1) * g.Hkv * rb].reshape(g.Hkv, rb)
        ro = ost[f"kv{p}"][y[1] * og.Hkv * rb:(y[1] + 1) * og.Hkv * rb].reshape(og.Hkv, rb)
        diff = (ra ^ ro) & bm
        if diff.any():
            h, byte = np.argwhere(diff)[0]
            raise AssertionError(f"b={b} entry {e} pool {p} head {h} byte {byte}: "
                                 f"gpu {ra[h, byte]:#x} oracle {ro[h, byte]:#x}")


def assert_sample_close(ref, got, sample, seq_len):
    out_ref, mass_ref, imp_ref = ref
    out, mass, imp = got
    for j, b in enumerate(sample):
        err = np.abs(out[b] - out_ref[j])
        lim = ATOL_OUT + RTOL_OUT * np.abs(out_ref[j])
        assert np.all(err <= lim), f"out b={b}: max err {err.max():.3g}"
        n = int(seq_len[b])
        e = np.abs(mass[b, :n] - mass_ref[j, :n])
        assert e.max(initial=0) <= ATOL_MASS, f"mass b={b}: max err {e.max():.3g}"
        if imp is not None:
            ei = np.abs(imp[b] - imp_ref[j])
            assert ei.max() <= ATOL_MASS, f"importance b={b}: max err {ei.max():.3g}"


def valid_positions(st: dict, g: wl.Geometry, b: int) -> np.ndarray:
    ps = [pp for (_, _, _, pos) in seq_layout(st, g, b) for pp in pos]
    return np.asarray(sorted(ps), dtype=np.int64)


def assert_properties(st: dict, g: wl.Geometry, got, Hq: int):
    """Properties of every sequence that hold at any size: finite output,
    mass zero at positions without a valid slot, mass sums to Hq, and the
    free stacks and tables partition every pool's ids."""
    out, mass, _ = got
    assert np.all(np.isfinite(out)), "non-finite output"
    for b in range(g.B):
        n = int(st["seq_len"][b])
        vp = valid_positions(st, g, b)
        hole = np.ones(n, dtype=bool)
        hole[vp] = False
        assert np.all(mass[b, :n][hole] == 0.0), f"mass at a hole b={b}"
        assert np.all(mass[b, n:] == -7.0), f"mass written past seq_len b={b}"
        if vp.size:
            s = float(mass[b, :n].astype(np.float64).sum())
            assert abs(s - Hq) <= 1e-3 * Hq, f"sum of mass b={b}: {s} (Hq={Hq})"
    assert_pools_partitioned(st, g)


def assert_pools_partitioned(st: dict, g: wl.Geometry):
    for p in range(3):
        top = int(st["free_top"][p])
        free = st[f"free{p}"][:top].astype(np.int64)
        used = []
        for b in range(g.B):
            nb = int(st["n_blocks"][b])
            row = st["table"][b * g.max_blocks: b * g.max_blocks + nb]
            used.append((row[(row >> 30) == p] & 0x3FFFFFFF).astype(np.int64))
        used = np.concatenate(used) if used else np.zeros(0, np.int64)
        allids = np.concatenate([free, used])
        assert allids.size == g.pool_blocks[p], f"pool {p}: {allids.size} ids for {g.pool_blocks[p]}"
        assert np.array_equal(np.sort(allids), np.arange(g.pool_blocks[p])), f"pool {p} ids not a partition"
