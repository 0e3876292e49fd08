"""Seeded synthetic inputs for thought-adaptive compressed-KV decode.

This module only draws random numbers and lays out an *empty* cache (zeroed
pools, empty block tables, free stacks in a seeded order).  It holds none of
the method's arithmetic: no quantisation, attention, mass or selection.  Both
the GPU library's tests/benchmark and the CPU oracle take their inputs from
here, so the two sides always see identical inputs.

Input recipe (stand-in for the long reasoning traces the pages evaluate on;
no dataset or model is used):
  * K, V ~ N(0, 1) rounded to fp16; in every kv head four key channels,
    chosen per workload, are multiplied by 10 before rounding (outliers).
  * q ~ N(0, 1) rounded to fp16.
  * Thought tags come in runs: run length ~ Geometric(1/32) (mean 32), run
    tag drawn i.i.d. with the workload's R/E/T probabilities
    ("ThinKV", Methodology, thought decomposition into R/E/T segments).
  * Eviction holes (long-trace workload): whole runs are dropped with
    probability 0.9 (T), 0.5 (E), 0.2 (R); then surviving runs are visited
    in random order and dropped with the same probabilities until at least
    60% of the tokens are gone.
  * Prior importance ~ Exponential(mean Hq/N) in fp32.
Every stream is a numpy PCG64 generator seeded by (workload id, sequence,
purpose), so any one sequence can be regenerated on its own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

HD = 128
BLK = 16
TAG_R, TAG_E, TAG_T = 0, 1, 2
TAG_SKIP = 255
SEED = 20261203


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload (shapes, tag mix, eviction settings)."""

    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    n_min: int                      # per-sequence cached tokens: fixed (n_min == n_max)
    n_max: int                      # or log-uniform in [n_min, n_max]
    tag_p: tuple = (0.3, 0.4, 0.3)  # R, E, T run probabilities
    identity_ids: bool = False      # physical block ids handed out 0, 1, 2, ...
    holes: float = 0.0              # >0: evict whole runs until this fraction is gone
    append_steps: int = 0           # tokens appended per sequence by the timed step
    importance: bool = False        # carries a prior importance buffer
    decay: float = 0.9
    keep: int = 0                   # fixed top-k per sequence (0: none)
    keep_frac: float = 0.0          # or keep max(keep_min, floor(frac * N))
    keep_min: int = 0
    q_window: int = 0
    recent_window: int = 0
    extra_steps: int = 64           # head-room for extra appended tokens
    period: int = 0                 # continuous-thinking loop: evict every `period` appends
    loop_steps: int = 0             # and run this many append+decode steps
    codec: int = 0                  # 1: ThinKV's FP8 / FP4 / ternary formats

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, Hq=8, Hkv=2, n_min=1024, n_max=1024,
                     identity_ids=True),
    "llama8b": Workload("llama8b", 1, B=16, Hq=32, Hkv=8, n_min=8192, n_max=8192),
    "long_evicted": Workload("long_evicted", 2, B=32, Hq=32, Hkv=8, n_min=32768,
                             n_max=32768, holes=0.6, append_steps=1),
    "budgeted": Workload("budgeted", 3, B=64, Hq=40, Hkv=8, n_min=16384, n_max=16384,
                         importance=True, keep=2048, q_window=64, recent_window=128),
    "ragged": Workload("ragged", 4, B=128, Hq=64, Hkv=8, n_min=1024, n_max=65536,
                       tag_p=(0.214, 0.286, 0.5), importance=True, keep_frac=0.05,
                       keep_min=256),
    # continuous thinking: a long generation under a fixed cache budget, the
    # cache pruned every `period` new tokens, so it oscillates between the
    # budget and budget + period ("TAM", periodic compaction)
    "ct_loop": Workload("ct_loop", 5, B=32, Hq=32, Hkv=8, n_min=4096, n_max=4096,
                        importance=True, keep=2048, q_window=64, recent_window=128,
                        period=256, loop_steps=4096, extra_steps=4096 + 64),
}


def scaled(w: Workload, **kw) -> Workload:
    """The same workload recipe at other sizes (for tests)."""
    return replace(w, **kw)


def _rng(w: Workload, *key) -> np.random.Generator:
    return np.random.default_rng([SEED, w.wid, *key])


def seq_lengths(w: Workload) -> np.ndarray:
    """Cached tokens per sequence (log-uniform when n_min < n_max)."""
    if w.n_min == w.n_max:
        return np.full(w.B, w.n_min, dtype=np.int64)
    u = _rng(w, 77777).uniform(math.log(w.n_min), math.log(w.n_max), size=w.B)
    return np.floor(np.exp(u)).astype(np.int64).clip(w.n_min, w.n_max)


def tag_runs(w: Workload, b: int, n: int):
    """Tags [n] (uint8) and the run each token belongs to (int32)."""
    rng = _rng(w, b, 1)
    tags = np.empty(n, dtype=np.uint8)
    run_id = np.empty(n, dtype=np.int32)
    i = r = 0
    while i < n:
        length = int(rng.geometric(1.0 / 32.0))
        tag = int(rng.choice(3, p=np.asarray(w.tag_p) / sum(w.tag_p)))
        j = min(n, i + length)
        tags[i:j] = tag
        run_id[i:j] = r
        i, r = j, r + 1
    return tags, run_id


def outlier_channels(w: Workload) -> np.ndarray:
    """[Hkv][4] key channels scaled by 10."""
    rng = _rng(w, 99998)
    return np.stack([rng.choice(HD, size=4, replace=False) for _ in range(w.Hkv)])


def token_kv(w: Workload, b: int, n: int):
    """K, V for n tokens of sequence b: fp16 [n][Hkv][128] each."""
    rng = _rng(w, b, 2)
    k = rng.standard_normal((n, w.Hkv, HD), dtype=np.float32)
    ch = outlier_channels(w)
    for h in range(w.Hkv):
        k[:, h, ch[h]] *= 10.0
    v = rng.standard_normal((n, w.Hkv, HD), dtype=np.float32)
    return k.astype(np.float16), v.astype(np.float16)


def queries(w: Workload, step: int = 0) -> np.ndarray:
    """q for one decode step: fp16 [B][Hq][128]."""
    return _rng(w, 99999, step).standard_normal((w.B, w.Hq, HD), dtype=np.float32).astype(np.float16)


def step_tokens(w: Workload, step: int):
    """New token per sequence for an appending step: (k, v fp16 [B][Hkv][128], tags [B])."""
    rng = _rng(w, 88888, step)
    k = rng.standard_normal((w.B, w.Hkv, HD), dtype=np.float32)
    ch = outlier_channels(w)
    for h in range(w.Hkv):
        k[:, h, ch[h]] *= 10.0
    v = rng.standard_normal((w.B, w.Hkv, HD), dtype=np.float32)
    tags = rng.choice(3, size=w.B, p=np.asarray(w.tag_p) / sum(w.tag_p)).astype(np.uint8)
    return k.astype(np.float16), v.astype(np.float16), tags


def loop_tags(w: Workload, n_total: int) -> np.ndarray:
    """Thought tags [B][n_total] of a generation that continues past the
    cached tokens: the same run process, drawn further (the first n tags of
    sequence b are tag_runs(w, b, n))."""
    return np.stack([tag_runs(w, b, n_total)[0] for b in range(w.B)])


def loop_step_tokens(w: Workload, step: int, tags_all: np.ndarray):
    """Token of loop step `step` for every sequence: k, v as step_tokens,
    with the tag at position (cached length + step) of the run stream."""
    k, v, _ = step_tokens(w, step)
    n = seq_lengths(w)
    return k, v, np.ascontiguousarray(tags_all[np.arange(w.B), n + step]).astype(np.uint8)


def keep_plan(w: Workload, b: int, tags: np.ndarray, run_id: np.ndarray) -> np.ndarray:
    """bool [n]: which cached tokens survive the planned eviction holes."""
    n = tags.size
    keep = np.ones(n, dtype=bool)
    if w.holes <= 0.0:
        return keep
    rng = _rng(w, b, 3)
    n_runs = int(run_id[-1]) + 1
    run_tag = np.zeros(n_runs, dtype=np.int64)
    run_tag[run_id] = tags
    p_drop = np.array([0.2, 0.5, 0.9])[run_tag]
    run_len = np.bincount(run_id, minlength=n_runs)
    alive = rng.random(n_runs) >= p_drop               # first pass over all runs
    gone = int(run_len[~alive].sum())
    target = w.holes * n
    while gone < target:                               # later passes stop at the target
        for r in rng.permutation(np.nonzero(alive)[0]):
            if rng.random() < p_drop[r]:
                alive[r] = False
                gone += int(run_len[r])
                if gone >= target:
                    break
    return alive[run_id]


def importance0(w: Workload, b: int, n_cap: int) -> np.ndarray:
    """Prior importance, fp32 [n_cap] ~ Exponential(mean Hq/N)."""
    n = int(seq_lengths(w)[b])
    return _rng(w, b, 4).exponential(w.Hq / n, size=n_cap).astype(np.float32)


def keep_counts(w: Workload) -> np.ndarray:
    """keep_k per sequence [B] (int32)."""
    n = seq_lengths(w)
    if w.keep_frac > 0:
        k = np.maximum(w.keep_min, np.floor(w.keep_frac * n)).astype(np.int32)
    else:
        k = np.full(w.B, w.keep, dtype=np.int32)
    return k


# --------------------------------------------------------------------------
# Empty cache layout
# --------------------------------------------------------------------------

def region_bytes(bits: int) -> int:
    """Bytes of one (block, kv head) region: K+V codes and their (scale, zero)."""
    return 512 * bits + 512


POOL_BITS = (8, 4, 2)


@dataclass
class Geometry:
    B: int
    Hq: int
    Hkv: int
    max_blocks: int
    n_cap: int
    pool_blocks: tuple
    codec: int = 0   # 0: integer min/max codes; 1: ThinKV's FP8 / FP4 / ternary formats

    def region_bytes(self, pool: int) -> int:
        return region_bytes(POOL_BITS[pool])


def geometry_for(w: Workload, all_tags: list | None = None, spare_per_seq: int = 4) -> Geometry:
    """Capacities large enough for the workload's cache plus its appended tokens."""
    n = seq_lengths(w)
    extra = w.extra_steps + w.append_steps
    max_blocks = int(math.ceil((int(n.max()) + extra) / BLK)) + 3 + spare_per_seq
    counts = np.zeros(3, dtype=np.int64)
    for b in range(w.B):
        tags = all_tags[b] if all_tags is not None else tag_runs(w, b, int(n[b]))[0]
        for p in range(3):
            counts[p] += int(math.ceil(int((tags == p).sum()) / BLK))
    spare = w.B * (spare_per_seq + int(math.ceil(extra / BLK)))
    pool_blocks = tuple(int(c + spare) for c in counts)
    return Geometry(w.B, w.Hq, w.Hkv, max_blocks, int(n.max()) + extra, pool_blocks, w.codec)


def empty_state(g: Geometry, identity_ids: bool, seed_key=(0,)) -> dict:
    """Host arrays of an empty cache.  Free stacks pop from the end; with
    identity_ids the pops hand out ids 0, 1, 2, ...; otherwise a seeded
    permutation."""
    st = {}
    for p in range(3):
        st[f"kv{p}"] = np.zeros(g.pool_blocks[p] * g.Hkv * g.region_bytes(p), dtype=np.uint8)
        st[f"mask{p}"] = np.zeros(g.pool_blocks[p], dtype=np.uint16)
        st[f"pos{p}"] = np.full(g.pool_blocks[p] * BLK, -1, dtype=np.int32)
        ids = np.arange(g.pool_blocks[p], dtype=np.uint32)
        if identity_ids:
            ids = ids[::-1].copy()
        else:
            ids = np.random.default_rng([SEED, 55555, *seed_key, p]).permutation(ids).astype(np.uint32)
        st[f"free{p}"] = ids
    st["table"] = np.zeros(g.B * g.max_blocks, dtype=np.uint32)
    st["n_blocks"] = np.zeros(g.B, dtype=np.int32)
    st["seq_len"] = np.zeros(g.B, dtype=np.int32)
    st["free_top"] = np.array(g.pool_blocks, dtype=np.int32)
    st["status"] = np.zeros(1, dtype=np.int32)
    return st


# --------------------------------------------------------------------------
# Per-workload token streams
# --------------------------------------------------------------------------

@dataclass
class Tokens:
    """All cached tokens of a workload, in lock-step (position-major) layout."""

    n: np.ndarray          # [B] cached tokens per sequence
    tags: np.ndarray       # [n_max][B] uint8 (TAG_SKIP past a sequence's end)
    k: np.ndarray          # [n_max][B][Hkv][128] fp16
    v: np.ndarray          # [n_max][B][Hkv][128] fp16
    keep: np.ndarray       # [B][n_cap] bool  planned survivors (holes workload)
    seq_tags: list = field(default_factory=list)


def lockstep_tokens(w: Workload, n_cap: int, threads: int = 8) -> Tokens:
    """Generate every cached token of every sequence (position-major)."""
    from concurrent.futures import ThreadPoolExecutor

    n = seq_lengths(w)
    n_max = int(n.max())
    tags = np.full((n_max, w.B), TAG_SKIP, dtype=np.uint8)
    k = np.zeros((n_max, w.B, w.Hkv, HD), dtype=np.float16)
    v = np.zeros((n_max, w.B, w.Hkv, HD), dtype=np.float16)
    keep = np.zeros((w.B, n_cap), dtype=bool)
    seq_tags = [None] * w.B

    def one(b):
        nb = int(n[b])
        t, run = tag_runs(w, b, nb)
        kb, vb = token_kv(w, b, nb)
        tags[:nb, b] = t
        k[:nb, b] = kb
        v[:nb, b] = vb
        keep[b, :nb] = keep_plan(w, b, t, run)
        seq_tags[b] = t

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(w.B)))
    return Tokens(n, tags, k, v, keep, seq_tags)
