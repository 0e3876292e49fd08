"""Thin ctypes binding of libkvq.so (include/kvq.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory and the stream.  If the library is
missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")
HD = 128

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_EHIP, KVQ_ENOSPC = 0, -1, -2, -3, -4
TAG_R, TAG_E, TAG_T, TAG_NONE = 0, 1, 2, 255

EXPORTS = ("kvq_region_bytes", "kvq_workspace_bytes", "kvq_decode_workspace_bytes", "kvq_append_quantize",
           "kvq_append_quantize_noalloc", "kvq_decode_attention", "kvq_evict_topk",
           "kvq_evict_tbe", "kvq_evict_tam")


class KvqError(RuntimeError):
    pass


class CacheStruct(ctypes.Structure):
    """struct kvq_cache."""
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("max_blocks", ctypes.c_int32), ("n_cap", ctypes.c_int32),
        ("pool_blocks", ctypes.c_int32 * 3), ("codec", ctypes.c_int32),
        ("kv", ctypes.c_void_p * 3), ("mask", ctypes.c_void_p * 3), ("pos", ctypes.c_void_p * 3),
        ("table", ctypes.c_void_p), ("n_blocks", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
        ("free_ids", ctypes.c_void_p * 3), ("free_top", ctypes.c_void_p), ("status", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """Load libkvq.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvqError(f"{LIB_PATH} not built (python -m eviction_kvq_decode_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, CS = ctypes.c_void_p, ctypes.POINTER(CacheStruct)
        L.kvq_region_bytes.restype = ctypes.c_size_t
        L.kvq_region_bytes.argtypes = [ctypes.c_int]
        L.kvq_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_workspace_bytes.argtypes = [CS]
        L.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_decode_workspace_bytes.argtypes = [CS]
        L.kvq_append_quantize.restype = ctypes.c_int
        L.kvq_append_quantize.argtypes = [CS, P, P, P, P, ctypes.c_size_t, P]
        L.kvq_append_quantize_noalloc.restype = ctypes.c_int
        L.kvq_append_quantize_noalloc.argtypes = [CS, P, P, P, P]
        L.kvq_decode_attention.restype = ctypes.c_int
        L.kvq_decode_attention.argtypes = [CS, P, P, P, P, ctypes.c_float, ctypes.c_float, P,
                                           ctypes.c_size_t, P]
        L.kvq_evict_topk.restype = ctypes.c_int
        L.kvq_evict_topk.argtypes = [CS, P, P, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_size_t, P]
        L.kvq_evict_tbe.restype = ctypes.c_int
        L.kvq_evict_tbe.argtypes = [CS, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, P, ctypes.c_size_t, P]
        L.kvq_evict_tam.restype = ctypes.c_int
        L.kvq_evict_tam.argtypes = [CS, P, P, ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    P, ctypes.c_size_t, P]
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != KVQ_OK:
        raise KvqError(f"{what} returned {rc}")


def _ptr(t):
    """Device address of a tensor (or an address passed as an int)."""
    if t is None or isinstance(t, int):
        return t
    return t.data_ptr()


class Cache:
    """A device-resident cache: torch tensors named as in
    workloads.empty_state, plus the kvq_cache struct that points at them."""

    def __init__(self, geometry, state: dict, device="cuda"):
        import torch

        self.g = geometry
        self.device = torch.device(device)
        self.t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(self.device) for k, v in state.items()}
        s = CacheStruct()
        g = geometry
        s.B, s.Hq, s.Hkv, s.head_dim = g.B, g.Hq, g.Hkv, HD
        s.max_blocks, s.n_cap = g.max_blocks, g.n_cap
        s.codec = getattr(g, "codec", 0)
        for p in range(3):
            s.pool_blocks[p] = g.pool_blocks[p]
            s.kv[p] = self.t[f"kv{p}"].data_ptr()
            s.mask[p] = self.t[f"mask{p}"].data_ptr()
            s.pos[p] = self.t[f"pos{p}"].data_ptr()
            s.free_ids[p] = self.t[f"free{p}"].data_ptr()
        s.table = self.t["table"].data_ptr()
        s.n_blocks = self.t["n_blocks"].data_ptr()
        s.seq_len = self.t["seq_len"].data_ptr()
        s.free_top = self.t["free_top"].data_ptr()
        s.status = self.t["status"].data_ptr()
        self.struct = s
        self.ws_bytes = lib().kvq_workspace_bytes(ctypes.byref(s))
        if self.ws_bytes == 0:
            raise KvqError("kvq_workspace_bytes rejected the cache geometry")
        # zero before the first call (the sync words of append and eviction)
        self.ws = torch.zeros(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self.ws.data_ptr()) % 256
        self.ws_ptr = self.ws.data_ptr() + off

    @staticmethod
    def _stream(stream):
        import torch

        return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream

    def append(self, k_new, v_new, tags, stream=None):
        """k_new, v_new: fp16 [B][Hkv][128]; tags: uint8 [B] (device tensors)."""
        _check(lib().kvq_append_quantize(ctypes.byref(self.struct), _ptr(k_new), _ptr(v_new),
                                         _ptr(tags), self.ws_ptr, self.ws_bytes,
                                         self._stream(stream)), "kvq_append_quantize")

    def append_noalloc(self, k_new, v_new, tags, stream=None):
        """kvq_append_quantize_noalloc: as append, with the library's static
        scratch instead of this cache's workspace."""
        _check(lib().kvq_append_quantize_noalloc(ctypes.byref(self.struct), _ptr(k_new), _ptr(v_new),
                                                 _ptr(tags), self._stream(stream)),
               "kvq_append_quantize_noalloc")

    def decode(self, q, out, mass, importance=None, decay=0.0, sm_scale=None, stream=None):
        """q fp16 [B][Hq][128]; out fp32 [B][Hq][128]; mass (and importance) fp32 [B][n_cap]."""
        if sm_scale is None:
            sm_scale = HD ** -0.5
        _check(lib().kvq_decode_attention(ctypes.byref(self.struct), _ptr(q), _ptr(out), _ptr(mass),
                                          _ptr(importance), float(decay), float(sm_scale),
                                          self.ws_ptr, self.ws_bytes, self._stream(stream)),
               "kvq_decode_attention")

    def evict(self, importance, keep_k, q_window, recent_window, stream=None):
        """importance fp32 [B][n_cap]; keep_k int32 [B]."""
        _check(lib().kvq_evict_topk(ctypes.byref(self.struct), _ptr(importance), _ptr(keep_k),
                                    int(q_window), int(recent_window), self.ws_ptr, self.ws_bytes,
                                    self._stream(stream)), "kvq_evict_topk")

    def evict_tbe(self, importance, r0, r_min, t_keep, q_window, recent_window, stream=None, seq_mask=None):
        """importance fp32 [B][n_cap]; thought-adaptive eviction by segment.
        seq_mask: uint8 [B] device tensor (or None: every sequence); the
        sequences outside it are left as they are."""
        _check(lib().kvq_evict_tbe(ctypes.byref(self.struct), _ptr(importance), _ptr(seq_mask), int(r0),
                                   int(r_min), int(t_keep), int(q_window), int(recent_window), self.ws_ptr,
                                   self.ws_bytes, self._stream(stream)), "kvq_evict_tbe")

    def evict_tam(self, score, keep_k, pivot_c, min_seg, q_window, recent_window, stream=None):
        """kvq_evict_tam: thought-aware segment budgets (score fp32 [B][n_cap],
        keep_k int32 [B], device tensors)."""
        _check(lib().kvq_evict_tam(ctypes.byref(self.struct), _ptr(score), _ptr(keep_k), float(pivot_c),
                                   int(min_seg), int(q_window), int(recent_window), self.ws_ptr,
                                   self.ws_bytes, self._stream(stream)), "kvq_evict_tam")

    def state_numpy(self) -> dict:
        """Host copy of every cache array (synchronises)."""
        return {k: v.cpu().numpy() for k, v in self.t.items()}

    @property
    def status(self) -> int:
        return int(self.t["status"].cpu()[0])
