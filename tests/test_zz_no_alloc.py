"""kvq_append_quantize_noalloc (static scratch, no workspace argument)
against kvq_append_quantize, through the C ABI: two calls in a row on
different caches, the second with a smaller batch, each compared bit for
bit (cache bytes and metadata) with the workspace entry point's result."""
import numpy as np
import pytest

from eviction_kvq_decode_amd import workloads as wl
from helpers import small_geometry
from pairs import log

pytestmark = pytest.mark.gpu

HD = 128


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _filled(g, rng, n):
    """A GPU cache after n lock-step appends (workspace entry point)."""
    from eviction_kvq_decode_amd import kvq

    c = kvq.Cache(g, wl.empty_state(g, identity_ids=False))
    for _ in range(n):
        k = rng.standard_normal((g.B, g.Hkv, HD)).astype(np.float16)
        v = rng.standard_normal((g.B, g.Hkv, HD)).astype(np.float16)
        c.append(_dev(k), _dev(v), _dev(rng.integers(0, 3, g.B).astype(np.uint8)))
    return c


def _one_call(B, n, seed):
    import torch

    from eviction_kvq_decode_amd import kvq

    log(f"[no-alloc] B={B} n={n}")
    g = small_geometry(B, 8, 2, n + 64)
    rng = np.random.default_rng(seed)
    ref = _filled(g, rng, n)
    torch.cuda.synchronize()
    got = kvq.Cache(g, ref.state_numpy())
    for step in range(3):
        k = _dev(rng.standard_normal((B, 2, HD)).astype(np.float16))
        v = _dev(rng.standard_normal((B, 2, HD)).astype(np.float16))
        # step 1: every sequence the same type (pops ranked across sequences);
        # one sequence skipped
        tags = rng.integers(0, 3, B).astype(np.uint8) if step != 1 else np.full(B, 2, np.uint8)
        tags[B // 2] = kvq.TAG_NONE if step == 2 else tags[B // 2]
        ref.append(k, v, _dev(tags))
        got.append_noalloc(k, v, _dev(tags))
        torch.cuda.synchronize()
        a, b = ref.state_numpy(), got.state_numpy()
        for key in a:
            assert np.array_equal(a[key], b[key]), f"{key} differs after step {step}"
    assert got.status == 0


def test_noalloc_append_matches_workspace_append():
    _one_call(40, 300, 1)
    _one_call(3, 120, 2)     # smaller batch into the same static scratch
