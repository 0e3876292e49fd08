"""Build the same cache on the oracle and on the GPU from one seeded workload,
and compare them.  Used by the GPU parity tests and the smoke check."""
from __future__ import annotations

import math
import sys
import time

import numpy as np

from eviction_kvq_decode_amd import workloads as wl
from oracle import oracle as orc

HD = 128
BLK = 16
# The five workload recipes at sizes the oracle finishes in seconds; each
# spans several table splits, partial blocks of every type and, for the
# ragged recipe, very different lengths.
SMALL_WORKLOADS = {
    "tiny": wl.WORKLOADS["tiny"],
    "llama8b": wl.scaled(wl.WORKLOADS["llama8b"], B=3, n_min=1500, n_max=1500),
    "long_evicted": wl.scaled(wl.WORKLOADS["long_evicted"], B=3, n_min=4100, n_max=4100),
    "budgeted": wl.scaled(wl.WORKLOADS["budgeted"], B=3, n_min=2600, n_max=2600, keep=300),
    "ragged": wl.scaled(wl.WORKLOADS["ragged"], B=5, n_min=40, n_max=5000, keep_min=24),
}

RTOL_OUT, ATOL_OUT = 2e-3, 1e-3    # attention output
ATOL_MASS = 1e-5                   # mass and importance


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Pair:
    """An oracle cache and a GPU cache holding the same workload."""

    def __init__(self, w: wl.Workload, want_gpu=True, step_tokens_dev=None):
        import torch

        from eviction_kvq_decode_amd import kvq

        self.w = w
        n = wl.seq_lengths(w)
        tmp_geo_cap = int(n.max()) + w.extra_steps + w.append_steps
        self.toks = wl.lockstep_tokens(w, tmp_geo_cap)
        self.g = wl.geometry_for(w, self.toks.seq_tags)
        assert self.g.n_cap == tmp_geo_cap
        state = wl.empty_state(self.g, w.identity_ids, seed_key=(w.wid,))
        self.oc = orc.OracleCache(self.g, state)
        self.gc = kvq.Cache(self.g, state) if want_gpu else None
        self.torch = torch

    def fill(self):
        """Lock-step appends of every cached token, then the planned holes."""
        torch = self.torch
        t0 = time.time()
        K = torch.from_numpy(self.toks.k).cuda()
        V = torch.from_numpy(self.toks.v).cuda()
        T = torch.from_numpy(self.toks.tags).cuda()
        for i in range(self.toks.k.shape[0]):
            self.oc.append(self.toks.k[i], self.toks.v[i], self.toks.tags[i])
            self.gc.append(K[i], V[i], T[i])
        torch.cuda.synchronize()
        del K, V, T
        if self.w.holes > 0:
            imp = self.toks.keep.astype(np.float32)
            keep_k = self.toks.keep.sum(axis=1).astype(np.int32)
            self.evict(imp, keep_k, 0, 0)
        log(f"  filled {self.w.name} B={self.w.B} in {time.time() - t0:.1f}s")

    def append_step(self, step=0):
        torch = self.torch
        k, v, tags = wl.step_tokens(self.w, step)
        self.oc.append(k, v, tags)
        self.gc.append(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(tags).cuda())

    def evict(self, imp, keep_k, qw, rw):
        torch = self.torch
        self.oc.evict(imp, keep_k, qw, rw)
        imp = np.ascontiguousarray(imp, dtype=np.float32)
        keep_k = np.ascontiguousarray(keep_k, dtype=np.int32)
        self.gc.evict(torch.from_numpy(imp).cuda(), torch.from_numpy(keep_k).cuda(), qw, rw)

    def decode(self, q, importance=None, decay=0.0):
        torch = self.torch
        g = self.g
        out_ref, mass_ref, imp_ref = self.oc.decode(q, 1 / math.sqrt(HD), importance, decay)
        out = torch.full((g.B, g.Hq, HD), float("nan"), device="cuda")
        mass = torch.full((g.B, g.n_cap), -7.0, device="cuda")
        imp_dev = None
        if importance is not None:
            imp_dev = torch.from_numpy(np.ascontiguousarray(importance, dtype=np.float32)).cuda()
        self.gc.decode(torch.from_numpy(q).cuda(), out, mass, imp_dev, decay)
        torch.cuda.synchronize()
        res = (out.cpu().numpy(), mass.cpu().numpy(), None if imp_dev is None else imp_dev.cpu().numpy())
        return (out_ref, mass_ref, imp_ref), res


# ---------------------------------------------------------------- compare

META = ("table", "n_blocks", "seq_len", "free_top", "status", "free0", "free1", "free2",
        "mask0", "mask1", "mask2")


def slot_byte_masks(bits: int) -> np.ndarray:
    """uint8 [16][region_bytes]: the bits of a region that belong to slot t."""
    rb = orc.region_bytes(bits)
    m = np.zeros((16, rb), dtype=np.uint8)
    lv = (1 << bits) - 1
    for t in range(16):
        m[t, t * 16 * bits:(t + 1) * 16 * bits] = 0xFF                      # K row
        m[t, 512 * bits + 16 * t: 512 * bits + 16 * t + 16] = 0xFF         # K (scale, zero)
        m[t, 512 * bits + 256 + 16 * t: 512 * bits + 256 + 16 * t + 16] = 0xFF
        for d in range(HD):
            bit = orc.v_bit_offset(bits, t, d)
            m[t, 256 * bits + bit // 8] |= np.uint8(lv << (bit % 8))
    return m


_SLOT_MASKS = {}


def assert_same_cache(oc, gst: dict, seqs=None):
    """Bit-exact comparison of all metadata and of every byte that belongs
    to a valid slot (the bytes of cleared slots are unspecified)."""
    for key in META:
        a, b = oc.st[key], gst[key]
        if key.startswith("free") and key != "free_top":
            p = int(key[-1])
            top = int(oc.st["free_top"][p])
            a, b = a[:top], b[:top]
        assert np.array_equal(a, b), f"{key} differs"
    # positions of valid slots
    for p in range(3):
        m = oc.st[f"mask{p}"]
        bits_set = ((m[:, None] >> np.arange(16)) & 1).astype(bool).ravel()
        assert np.array_equal(oc.st[f"pos{p}"][bits_set], gst[f"pos{p}"][bits_set]), f"pos{p}"
    g = oc.g
    for p, bits in enumerate((8, 4, 2)):
        if bits not in _SLOT_MASKS:
            _SLOT_MASKS[bits] = slot_byte_masks(bits)
        sm = _SLOT_MASKS[bits]
        rb = orc.region_bytes(bits)
        mask = oc.st[f"mask{p}"]
        ids = np.nonzero(mask)[0]
        if seqs is not None:
            keep = set()
            for b in seqs:
                for ent in oc.table_row(b):
                    if ent >> 30 == p:
                        keep.add(int(ent & 0x3FFFFFFF))
            ids = np.array(sorted(keep), dtype=np.int64)
        if ids.size == 0:
            continue
        bm = np.zeros((ids.size, rb), dtype=np.uint8)
        for t in range(16):
            sel = ((mask[ids] >> t) & 1).astype(bool)
            bm[sel] |= sm[t]
        A = oc.st[f"kv{p}"].reshape(-1, g.Hkv, rb)[ids]
        Bv = gst[f"kv{p}"].reshape(-1, g.Hkv, rb)[ids]
        diff = (A ^ Bv) & bm[:, None, :]
        if diff.any():
            i, h, byte = np.argwhere(diff)[0]
            raise AssertionError(f"pool {p} block {ids[i]} head {h} byte {byte}: "
                                 f"oracle {A[i, h, byte]:#x} gpu {Bv[i, h, byte]:#x}")


def assert_attention_close(ref, got, valid_mass_only=True, seqs=None):
    out_ref, mass_ref, imp_ref = ref
    out, mass, imp = got
    B = out.shape[0]
    seqs = range(B) if seqs is None else seqs
    for b in seqs:
        err = np.abs(out[b] - out_ref[b])
        lim = ATOL_OUT + RTOL_OUT * np.abs(out_ref[b])
        assert np.all(err <= lim), f"out b={b}: max err {err.max():.3g} (worst excess {(err - lim).max():.3g})"
    return True


def assert_mass_close(seq_len, ref, got, seqs=None):
    _, mass_ref, imp_ref = ref
    _, mass, imp = got
    seqs = range(mass.shape[0]) if seqs is None else seqs
    for b in seqs:
        n = int(seq_len[b])
        e = np.abs(mass[b, :n] - mass_ref[b, :n])
        assert e.max(initial=0) <= ATOL_MASS, f"mass b={b}: max err {e.max():.3g}"
        assert np.all(mass[b, n:] == -7.0), "mass written past seq_len"
        if imp is not None:
            ei = np.abs(imp[b] - imp_ref[b])
            assert ei.max() <= ATOL_MASS, f"importance b={b}: max err {ei.max():.3g}"
