"""ctypes front end of the CPU oracle (kvq_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  See kvq_oracle.c for what
it computes and which page section each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")
HD = 128
BLK = 16
POOL_BITS = (8, 4, 2)

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-o", LIB_PATH + ".tmp", SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Cache(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32), ("n_cap", ctypes.c_int32),
        ("pool_blocks", ctypes.c_int32 * 3), ("codec", ctypes.c_int32),
        ("kv", ctypes.c_void_p * 3), ("mask", ctypes.c_void_p * 3), ("pos", ctypes.c_void_p * 3),
        ("table", ctypes.c_void_p), ("n_blocks", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
        ("free_ids", ctypes.c_void_p * 3), ("free_top", ctypes.c_void_p), ("status", ctypes.c_void_p),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.orc_half_to_double.restype = ctypes.c_double
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_float_to_half.restype = ctypes.c_uint16
        L.orc_float_to_half.argtypes = [ctypes.c_float]
        L.orc_half_to_double_array.argtypes = [P, P, ctypes.c_long]
        L.orc_float_to_half_array.argtypes = [P, P, ctypes.c_long]
        L.orc_quantize_groups.argtypes = [P, ctypes.c_long, ctypes.c_int, P, P, P]
        L.orc_quantize_groups_native.argtypes = [P, ctypes.c_long, ctypes.c_int, P, P, P]
        L.orc_native_values.argtypes = [ctypes.c_int, P, ctypes.c_long, P]
        L.orc_mini_encode_array.argtypes = [P, ctypes.c_long, ctypes.c_int, P]
        L.orc_k_row_index.restype = ctypes.c_int
        L.orc_k_row_index.argtypes = [ctypes.c_int, ctypes.c_int]
        L.orc_k_bit_offset.restype = ctypes.c_long
        L.orc_k_bit_offset.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.orc_v_bit_offset.restype = ctypes.c_long
        L.orc_v_bit_offset.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.orc_region_bytes.restype = ctypes.c_long
        L.orc_region_bytes.argtypes = [ctypes.c_int]
        L.orc_append.argtypes = [ctypes.POINTER(_Cache), P, P, P]
        L.orc_decode.argtypes = [ctypes.POINTER(_Cache), P, ctypes.c_double, P, P, P, P,
                                 ctypes.c_double, P]
        L.orc_evict.argtypes = [ctypes.POINTER(_Cache), P, P, ctypes.c_int, ctypes.c_int]
        L.orc_evict_tbe.argtypes = [ctypes.POINTER(_Cache), P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int]
        L.orc_evict_tam.argtypes = [ctypes.POINTER(_Cache), P, P, ctypes.c_float, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int]
        L.orc_dequant_slot.argtypes = [ctypes.POINTER(_Cache), ctypes.c_int, ctypes.c_uint32,
                                       ctypes.c_int, ctypes.c_int, P, P]
        L.orc_slot_codes.argtypes = [ctypes.POINTER(_Cache), ctypes.c_int, ctypes.c_uint32,
                                     ctypes.c_int, ctypes.c_int, P, P, P, P]
        L.orc_put_slot_codes.argtypes = [ctypes.POINTER(_Cache), ctypes.c_int, ctypes.c_uint32,
                                         ctypes.c_int, ctypes.c_int, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


# ---------------------------------------------------------------- scalars

def half_to_double(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    lib().orc_half_to_double_array(_p(h), _p(out), h.size)
    return out


def float_to_half(f: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    lib().orc_float_to_half_array(_p(f), _p(out), f.size)
    return out


def quantize_groups(x_fp16: np.ndarray, bits: int):
    """x: fp16 [..., 32] -> (scale bits [...], zero bits [...], codes uint8 [..., 32])."""
    x = np.ascontiguousarray(x_fp16, dtype=np.float16).view(np.uint16)
    assert x.shape[-1] == 32
    ng = x.size // 32
    sc = np.empty(x.shape[:-1], dtype=np.uint16)
    zr = np.empty(x.shape[:-1], dtype=np.uint16)
    codes = np.empty(x.shape, dtype=np.uint8)
    lib().orc_quantize_groups(_p(x), ng, bits, _p(sc), _p(zr), _p(codes))
    return sc, zr, codes


def quantize_groups_native(x_fp16: np.ndarray, pool: int):
    """ThinKV's formats (pool 0 E4M3, 1 E2M1, 2 ternary): x fp16 [..., 32] ->
    (scale bits, zero bits, codes)."""
    x = np.ascontiguousarray(x_fp16, dtype=np.float16).view(np.uint16)
    assert x.shape[-1] == 32
    sc = np.empty(x.shape[:-1], dtype=np.uint16)
    zr = np.empty(x.shape[:-1], dtype=np.uint16)
    codes = np.empty(x.shape, dtype=np.uint8)
    lib().orc_quantize_groups_native(_p(x), x.size // 32, int(pool), _p(sc), _p(zr), _p(codes))
    return sc, zr, codes


def native_values(pool: int, codes: np.ndarray) -> np.ndarray:
    """Values of E4M3 (pool 0) or E2M1 (pool 1) codes, before the scale."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().orc_native_values(int(pool), _p(c), c.size, _p(out))
    return out


def mini_encode(y: np.ndarray, pool: int) -> np.ndarray:
    """Nearest E4M3 (pool 0) or E2M1 (pool 1) code of fp32 values."""
    yy = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(yy.shape, dtype=np.uint8)
    lib().orc_mini_encode_array(_p(yy), yy.size, int(pool), _p(out))
    return out


def k_bit_offset(bits: int, t: int, d: int) -> int:
    return lib().orc_k_bit_offset(bits, t, d)


def v_bit_offset(bits: int, t: int, d: int) -> int:
    return lib().orc_v_bit_offset(bits, t, d)


def region_bytes(bits: int) -> int:
    return lib().orc_region_bytes(bits)


# ---------------------------------------------------------------- cache

class OracleCache:
    """Host copy of a cache, driven by the oracle.  `state` holds the arrays
    named as in workloads.empty_state (copied on construction)."""

    def __init__(self, geometry, state: dict):
        self.g = geometry
        self.st = {k: np.array(v, copy=True) for k, v in state.items()}
        self._struct = None

    def _c(self):
        s = _Cache()
        g, st = self.g, self.st
        s.B, s.Hq, s.Hkv, s.max_blocks, s.n_cap = g.B, g.Hq, g.Hkv, g.max_blocks, g.n_cap
        s.codec = getattr(g, "codec", 0)
        for p in range(3):
            s.pool_blocks[p] = g.pool_blocks[p]
            s.kv[p] = _p(st[f"kv{p}"])
            s.mask[p] = _p(st[f"mask{p}"])
            s.pos[p] = _p(st[f"pos{p}"])
            s.free_ids[p] = _p(st[f"free{p}"])
        s.table = _p(st["table"])
        s.n_blocks = _p(st["n_blocks"])
        s.seq_len = _p(st["seq_len"])
        s.free_top = _p(st["free_top"])
        s.status = _p(st["status"])
        self._struct = s  # keep alive
        return ctypes.byref(s)

    # -- the three operations -------------------------------------------
    def append(self, k_new: np.ndarray, v_new: np.ndarray, tags: np.ndarray):
        k = np.ascontiguousarray(k_new, dtype=np.float16).view(np.uint16)
        v = np.ascontiguousarray(v_new, dtype=np.float16).view(np.uint16)
        t = np.ascontiguousarray(tags, dtype=np.uint8)
        assert k.shape == (self.g.B, self.g.Hkv, HD) and t.shape == (self.g.B,)
        lib().orc_append(self._c(), _p(k), _p(v), _p(t))

    def decode(self, q: np.ndarray, sm_scale: float, importance: np.ndarray | None = None,
               decay: float = 0.0, want: np.ndarray | None = None):
        """Returns (out fp64 [B][Hq][128], mass fp64 [B][n_cap], importance' fp32 or None)."""
        g = self.g
        qq = np.ascontiguousarray(q, dtype=np.float16).view(np.uint16)
        assert qq.shape == (g.B, g.Hq, HD)
        out = np.zeros((g.B, g.Hq, HD), dtype=np.float64)
        mass = np.zeros((g.B, g.n_cap), dtype=np.float64)
        imp_in = imp_out = None
        if importance is not None:
            imp_in = np.ascontiguousarray(importance, dtype=np.float32).reshape(g.B, g.n_cap)
            imp_out = np.empty_like(imp_in)
        w = None if want is None else np.ascontiguousarray(want, dtype=np.uint8)
        lib().orc_decode(self._c(), _p(qq), float(sm_scale), _p(out), _p(mass), _p(imp_in),
                         _p(imp_out), float(decay), _p(w))
        return out, mass, imp_out

    def evict(self, importance: np.ndarray, keep_k: np.ndarray, q_window: int, recent_window: int):
        g = self.g
        imp = np.ascontiguousarray(importance, dtype=np.float32).reshape(g.B, g.n_cap)
        kk = np.ascontiguousarray(keep_k, dtype=np.int32)
        assert kk.shape == (g.B,)
        lib().orc_evict(self._c(), _p(imp), _p(kk), int(q_window), int(recent_window))

    def evict_tbe(self, importance: np.ndarray, r0: int, r_min: int, t_keep: int, q_window: int,
                  recent_window: int, seq_mask=None):
        """Thought-adaptive eviction ("ThinKV", think-before-evict); see
        orc_evict_tbe in kvq_oracle.c.  seq_mask: uint8 [B] (None: every
        sequence); the sequences outside it are skipped."""
        g = self.g
        imp = np.ascontiguousarray(importance, dtype=np.float32).reshape(g.B, g.n_cap)
        sm = None if seq_mask is None else np.ascontiguousarray(seq_mask, dtype=np.uint8).reshape(g.B)
        lib().orc_evict_tbe(self._c(), _p(imp), None if sm is None else _p(sm), int(r0), int(r_min),
                            int(t_keep), int(q_window), int(recent_window))

    def evict_tam(self, score: np.ndarray, keep_k, pivot_c: float, min_seg: int, q_window: int,
                  recent_window: int):
        """Thought-aware budgets ("TAM", section 2: segments, sqrt(w) n
        budgets, pivotal tokens); see orc_evict_tam in kvq_oracle.c."""
        g = self.g
        sc = np.ascontiguousarray(score, dtype=np.float32).reshape(g.B, g.n_cap)
        kk = np.ascontiguousarray(np.broadcast_to(np.asarray(keep_k, dtype=np.int32), (g.B,)))
        lib().orc_evict_tam(self._c(), _p(sc), _p(kk), float(pivot_c), int(min_seg), int(q_window),
                            int(recent_window))

    # -- inspection -----------------------------------------------------
    @property
    def status(self) -> int:
        return int(self.st["status"][0])

    def table_row(self, b: int) -> np.ndarray:
        n = int(self.st["n_blocks"][b])
        return self.st["table"][b * self.g.max_blocks: b * self.g.max_blocks + n].copy()

    def valid_slots(self, b: int):
        """[(pool, id, slot, pos)] in table order, then slot order."""
        out = []
        for ent in self.table_row(b):
            pool, bid = int(ent >> 30), int(ent & 0x3FFFFFFF)
            m = int(self.st[f"mask{pool}"][bid])
            for s in range(BLK):
                if (m >> s) & 1:
                    out.append((pool, bid, s, int(self.st[f"pos{pool}"][bid * BLK + s])))
        return out

    def slot_codes(self, pool: int, bid: int, h: int, t: int):
        kc = np.empty(HD, np.uint8)
        vc = np.empty(HD, np.uint8)
        ks = np.empty(8, np.uint16)
        vs = np.empty(8, np.uint16)
        lib().orc_slot_codes(self._c(), pool, bid, h, t, _p(kc), _p(vc), _p(ks), _p(vs))
        return kc, vc, ks, vs

    def put_slot_codes(self, pool: int, bid: int, h: int, t: int, kc, vc):
        kc = np.ascontiguousarray(kc, dtype=np.uint8)
        vc = np.ascontiguousarray(vc, dtype=np.uint8)
        lib().orc_put_slot_codes(self._c(), pool, bid, h, t, _p(kc), _p(vc))

    def dequant_slot(self, pool: int, bid: int, h: int, t: int):
        k = np.empty(HD, np.float64)
        v = np.empty(HD, np.float64)
        lib().orc_dequant_slot(self._c(), pool, bid, h, t, _p(k), _p(v))
        return k, v
