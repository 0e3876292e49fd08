"""The C-ABI library loads, exports every entry point include/kvq.h declares,
and rejects bad host-side arguments without touching a GPU."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from eviction_kvq_decode_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|kvq_status)\s+(kvq_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(kvq.EXPORTS)
    L = kvq.lib()
    for n in names:
        assert hasattr(L, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", nm, re.M), n


def test_boundary_calls_exported():
    """The calls the hot path's boundary is drawn with: append + quantise,
    the decode with its workspace size, windowed top-k eviction."""
    L = kvq.lib()
    for n in ("kvq_append_quantize", "kvq_decode_workspace_bytes", "kvq_decode_attention", "kvq_evict_topk"):
        assert n in _declared() and hasattr(L, n), n


def test_struct_layout_matches_header(tmp_path):
    fields = [f[0] for f in kvq.CacheStruct._fields_]
    prog = tmp_path / "layout.c"
    body = "".join(f'printf("{f} %zu\\n", offsetof(kvq_cache, {f}));\n' for f in fields)
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "kvq.h"\nint main(void){\n'
                    + body + 'printf("size %zu\\n", sizeof(kvq_cache));\nreturn 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(prog), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(out[f]) == getattr(kvq.CacheStruct, f).offset, f
    assert int(out["size"]) == ctypes.sizeof(kvq.CacheStruct)


def _dummy_struct(**over):
    s = kvq.CacheStruct()
    s.B, s.Hq, s.Hkv, s.head_dim, s.max_blocks, s.n_cap = 2, 8, 2, 128, 16, 256
    for p in range(3):
        s.pool_blocks[p] = 32
        s.kv[p] = s.mask[p] = s.pos[p] = s.free_ids[p] = 0x1000
    s.table = s.n_blocks = s.seq_len = s.free_top = s.status = 0x1000
    for k, v in over.items():
        setattr(s, k, v)
    return s


def test_region_and_workspace_sizes():
    L = kvq.lib()
    assert [L.kvq_region_bytes(p) for p in range(3)] == [4608, 2560, 1536]
    assert L.kvq_region_bytes(3) == 0
    s = _dummy_struct()
    ws = L.kvq_workspace_bytes(ctypes.byref(s))
    # decode partials + per-slot scores dominate
    assert ws >= 4 * 2 * 8 * 16 * 16
    assert L.kvq_workspace_bytes(ctypes.byref(_dummy_struct(head_dim=64))) == 0


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=64), kvq.KVQ_EUNSUPPORTED),
    (dict(Hq=34, Hkv=2), kvq.KVQ_EUNSUPPORTED),      # GQA group of 17
    (dict(Hq=9, Hkv=2), kvq.KVQ_EINVAL),
    (dict(B=0), kvq.KVQ_EINVAL),
    (dict(table=None), kvq.KVQ_EINVAL),
    (dict(codec=2), kvq.KVQ_EINVAL),
])
def test_host_side_validation(over, code):
    L = kvq.lib()
    s = _dummy_struct(**over)
    buf = 0x100000
    assert L.kvq_append_quantize(ctypes.byref(s), buf, buf, buf, buf, 1 << 40, None) == code
    assert L.kvq_append_quantize_noalloc(ctypes.byref(s), buf, buf, buf, None) == code
    assert L.kvq_decode_attention(ctypes.byref(s), buf, buf, buf, None, 0.9, 0.1, buf, 1 << 40, None) == code
    assert L.kvq_evict_topk(ctypes.byref(s), buf, buf, 0, 0, buf, 1 << 40, None) == code
    assert L.kvq_evict_tbe(ctypes.byref(s), buf, None, 64, 1, 4, 0, 0, buf, 1 << 40, None) == code
    assert L.kvq_evict_tam(ctypes.byref(s), buf, buf, 2.0, 1, 0, 0, buf, 1 << 40, None) == code


def test_bad_arguments_rejected_before_launch():
    L = kvq.lib()
    s = _dummy_struct()
    ok = 0x100000
    need = L.kvq_workspace_bytes(ctypes.byref(s))
    dneed = L.kvq_decode_workspace_bytes(ctypes.byref(s))
    assert 0 < dneed <= need
    # each call checks the workspace against its own need
    assert L.kvq_decode_attention(ctypes.byref(s), ok, ok, ok, None, 0.9, 0.1, ok, dneed - 1, None) == \
        kvq.KVQ_EINVAL
    assert L.kvq_append_quantize(ctypes.byref(s), None, ok, ok, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_append_quantize(ctypes.byref(s), ok, ok, ok, ok, 255, None) == kvq.KVQ_EINVAL
    assert L.kvq_append_quantize(ctypes.byref(s), ok, ok, ok, ok + 8, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_append_quantize_noalloc(ctypes.byref(s), None, ok, ok, None) == kvq.KVQ_EINVAL
    assert L.kvq_append_quantize_noalloc(ctypes.byref(s), ok, ok, None, None) == kvq.KVQ_EINVAL
    assert L.kvq_append_quantize_noalloc(ctypes.byref(_dummy_struct(B=1025)), ok, ok, ok, None) == \
        kvq.KVQ_EUNSUPPORTED
    assert L.kvq_decode_attention(ctypes.byref(s), ok, None, ok, None, 0.9, 0.1, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_topk(ctypes.byref(s), ok, ok, -1, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_topk(ctypes.byref(s), None, ok, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tbe(ctypes.byref(s), None, None, 64, 1, 4, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tbe(ctypes.byref(s), ok, None, -1, 1, 4, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tbe(ctypes.byref(s), ok, None, 64, 1, -4, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tbe(ctypes.byref(s), ok, None, 64, 1, 4, 0, -1, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tbe(ctypes.byref(s), ok, None, 64, 1, 4, 0, 0, ok, 255, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tam(ctypes.byref(s), None, ok, 2.0, 1, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tam(ctypes.byref(s), ok, None, 2.0, 1, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tam(ctypes.byref(s), ok, ok, -1.0, 1, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tam(ctypes.byref(s), ok, ok, float("nan"), 1, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tam(ctypes.byref(s), ok, ok, 2.0, 0, 0, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tam(ctypes.byref(s), ok, ok, 2.0, 1, -1, 0, ok, need, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_tam(ctypes.byref(s), ok, ok, 2.0, 1, 0, 0, ok, 255, None) == kvq.KVQ_EINVAL
    assert L.kvq_evict_topk(ctypes.byref(s), ok, ok, 0, 0, ok, 255, None) == kvq.KVQ_EINVAL
