"""Benchmark: decode attention over the compressed, partly evicted KV cache.

One step = append one new token per sequence (quantise into a free slot of
its type) + decode attention for one query token per sequence (output,
per-position mass), on the long-reasoning-trace workload:
B=32, Hq=32, Hkv=8, D=128, 32768 logical positions per sequence, 60% of the
slots evicted (whole thought runs, T-biased), tokens at 8/4/2 bits by type.

Prints one JSON line.  `value` is decode tokens/s (B tokens per step);
`roofline` rates the decode call against MI355X HBM bandwidth on the
compressed-KV bytes it must read; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--no-cpu] [--workload NAME]

--workload budgeted (or another workload with an eviction budget) times the
eviction step instead: decode with importance accumulation + windowed top-k
evict, and reports the evict call beside the decode roofline.
--workload ct_loop runs the continuous-thinking loop (a long generation
under a cache budget, pruned every P tokens) and reports time per step and
the cache footprint.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn tokens/s + effective compressed-KV GB/s (% of HBM peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
# segment-granular eviction timed beside top-k: retention 64 for a segment
# with one later Transition segment, halved per further one down to 4, and
# 8 tokens kept of each earlier Transition segment ("ThinKV", Methodology,
# think-before-evict: 64, 32, 16, ... as its example schedule)
TBE_PARAMS = (64, 4, 8)
# thought-aware budgets timed beside them: the workload's keep as the budget,
# the importance as the window score, pivotal above 8x the mean, runs
# shorter than 16 candidates merged ("TAM", section 2)
TAM_PARAMS = (8.0, 16)
# the continuous-thinking loop's TAM pruning: the same, on the mass of the
# last 64 queries before each prune (the selection window, "TAM", 2.B)
CT_TAM_PARAMS = TAM_PARAMS + (64,)
# the arithmetic of the path: codes widened to exact fp16 MFMA operands
# against fp16 q / P', accumulated in fp32; softmax, mass and the merge in fp32
DTYPE = "fp16-mfma/fp32-acc"
# rotate cache copies until they hold at least this many bytes (2x the MALL)
MALL_ROTATE_BYTES = 512e6
DECODE_KERNEL = "kvq_decode_attention (split + finalize)"
ROW_BYTES = (288, 160, 96)   # K+V codes + (scale, zero) per token per kv head, R/E/T


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kv_bytes(tags_valid: np.ndarray, Hkv: int) -> int:
    return int(np.asarray(ROW_BYTES)[tags_valid.astype(np.int64)].sum()) * Hkv


def build_gpu_cache(w, toks, g):
    import torch

    from eviction_kvq_decode_amd import kvq
    from eviction_kvq_decode_amd import workloads as wl

    cache = kvq.Cache(g, wl.empty_state(g, w.identity_ids, seed_key=(w.wid,)))
    K = torch.from_numpy(toks.k).cuda()
    V = torch.from_numpy(toks.v).cuda()
    T = torch.from_numpy(toks.tags).cuda()
    sk, sv, st = K[0].numel() * 2, V[0].numel() * 2, T[0].numel()
    kp, vp, tp = K.data_ptr(), V.data_ptr(), T.data_ptr()
    for i in range(toks.k.shape[0]):
        cache.append(kp + i * sk, vp + i * sv, tp + i * st)
    torch.cuda.synchronize()
    del K, V, T
    if w.holes > 0:
        imp = torch.from_numpy(toks.keep.astype(np.float32)).cuda()
        keep = torch.from_numpy(toks.keep.sum(axis=1).astype(np.int32)).cuda()
        cache.evict(imp, keep, 0, 0)
    torch.cuda.synchronize()
    if cache.status != 0:
        raise RuntimeError(f"cache build set status {cache.status}")
    return cache


def valid_slot_count(cache) -> int:
    """Valid slots of all table entries of all sequences (host copy of the
    metadata only)."""
    g = cache.g
    nb = cache.t["n_blocks"].cpu().numpy()
    table = cache.t["table"].cpu().numpy().reshape(g.B, g.max_blocks)
    masks = [cache.t[f"mask{p}"].cpu().numpy().astype(np.int64) for p in range(3)]
    total = 0
    for b in range(g.B):
        ent = table[b, : nb[b]].astype(np.int64)
        pool, bid = ent >> 30, ent & 0x3FFFFFFF
        for p in range(3):
            m = masks[p][bid[pool == p]]
            total += int(sum(bin(int(x)).count("1") for x in m))
    return total


def committed_traffic(workload: str):
    """HBM bytes per decode call from the committed FETCH_SIZE / WRITE_SIZE
    measurement (profiles/decode_long_evicted_traffic.json), or None when it
    does not cover this workload or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "decode_long_evicted_traffic.json")
    if workload != "long_evicted" or not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    h = hashlib.sha256()
    for src in d["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return d["hbm_bytes_per_call"] if h.hexdigest() == d["sources_sha256"] else None


TRAFFIC_SOURCES = ["eviction_kvq_decode_amd/csrc/kvq_attn.hip", "eviction_kvq_decode_amd/csrc/kvq_internal.h",
                   "eviction_kvq_decode_amd/csrc/kvq_device.h"]


def traffic_record(fetch_csv: str, write_csv: str, copy_mb: int) -> dict:
    """The committed traffic record from two rocprofv3 --pmc runs of this
    script (FETCH_SIZE, then WRITE_SIZE, each with --copy-probe-mb copy_mb):
    per-dispatch KiB of the decode kernels, scaled by what the same counter
    reads for the probe's copies (copy_mb MiB read and written each)."""
    import csv
    from collections import defaultdict

    def means(path, counter):
        vals = defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                key = ("copy" if "copyBuffer" in name else "split" if "attn_split" in name
                       else "finalize" if "attn_finalize" in name else None)
                if key:
                    vals[key].append(float(row["Counter_Value"]))
        probe = sorted(vals["copy"])[-3:]   # the three probe copies are the largest
        return {k: float(np.mean(v)) for k, v in vals.items() if k != "copy"}, float(np.mean(probe))

    copy_bytes = copy_mb << 20
    fetch, fetch_copy = means(fetch_csv, "FETCH_SIZE")
    write, write_copy = means(write_csv, "WRITE_SIZE")
    rs, ws = copy_bytes / (fetch_copy * 1024), copy_bytes / (write_copy * 1024)
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    rd = (fetch["split"] + fetch["finalize"]) * 1024 * rs
    wr = (write["split"] + write["finalize"]) * 1024 * ws
    return {"workload": "long_evicted: B=32 Hq=32 Hkv=8 D=128, 32768 positions, 60% evicted",
            "kernel": "kvq_decode_attention (attn_split + attn_finalize)",
            "sources_sha256": h.hexdigest(), "sources": TRAFFIC_SOURCES,
            "copy_probe_bytes": copy_bytes, "fetch_kib_per_copy": fetch_copy, "write_kib_per_copy": write_copy,
            "read_scale": rs, "write_scale": ws,
            "split_fetch_kib": fetch["split"], "split_write_kib": write["split"],
            "finalize_fetch_kib": fetch["finalize"], "finalize_write_kib": write["finalize"],
            "hbm_read_bytes": rd, "hbm_write_bytes": wr, "hbm_bytes_per_call": rd + wr}


def host_cpu(units: int) -> dict:
    """The host the oracle runs on: cores this process may use, the CPU
    model, and the OpenMP threads the oracle's decode can keep busy (it runs
    over (sequence, kv head) pairs, `units` of them)."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    omp = int(os.environ.get("OMP_NUM_THREADS", nproc))
    return {"nproc": nproc, "model": model, "threads": max(1, min(omp, units))}


def cpu_baseline(w, toks, n_seq: int, seconds: float):
    """Time the CPU oracle on the first n_seq sequences of the workload."""
    from eviction_kvq_decode_amd import workloads as wl
    from oracle import oracle as orc

    ws = wl.scaled(w, B=n_seq)
    g = wl.geometry_for(ws, toks.seq_tags[:n_seq])
    oc = orc.OracleCache(g, wl.empty_state(g, ws.identity_ids, seed_key=(w.wid,)))
    t0 = time.time()
    for i in range(toks.k.shape[0]):
        oc.append(toks.k[i, :n_seq], toks.v[i, :n_seq], toks.tags[i, :n_seq])
    if w.holes > 0:
        keep = toks.keep[:n_seq]
        oc.evict(keep.astype(np.float32), keep.sum(axis=1).astype(np.int32), 0, 0)
    log(f"[cpu] oracle sample of {n_seq} sequences built in {time.time() - t0:.1f}s")
    reps, t0 = 0, time.time()
    step = 0
    while time.time() - t0 < seconds or reps < 2:
        k, v, tags = wl.step_tokens(w, 10_000 + step)
        oc.append(k[:n_seq], v[:n_seq], tags[:n_seq])
        oc.decode(wl.queries(w, step)[:n_seq], 1 / math.sqrt(128))
        reps += 1
        step += 1
    dt = time.time() - t0
    hc = host_cpu(n_seq * w.Hkv)
    return {"value": n_seq * reps / dt, "unit": "tokens/s", "cores": hc["threads"],
            "kind": "oracle", "nproc": hc["nproc"], "cpu_model": hc["model"],
            "sample": f"{n_seq} of {w.B} sequences at full length, {reps} append+decode steps "
                      f"in {dt:.1f}s (fp64 C, OpenMP over (sequence, kv head) pairs)"}


def cpu_baseline_evict(w, toks, n_seq: int, seconds: float):
    """Time the CPU oracle's decode (with importance) + top-k evict on the
    first n_seq sequences, restoring the cache state before each step."""
    import copy

    from eviction_kvq_decode_amd import workloads as wl
    from oracle import oracle as orc

    ws = wl.scaled(w, B=n_seq)
    g = wl.geometry_for(ws, toks.seq_tags[:n_seq])
    oc = orc.OracleCache(g, wl.empty_state(g, ws.identity_ids, seed_key=(w.wid,)))
    for i in range(toks.k.shape[0]):
        oc.append(toks.k[i, :n_seq], toks.v[i, :n_seq], toks.tags[i, :n_seq])
    st0 = copy.deepcopy(oc.st)
    imp0 = np.stack([wl.importance0(w, b, g.n_cap) for b in range(n_seq)])
    keep_k = wl.keep_counts(w)[:n_seq]
    reps, busy = 0, 0.0
    while busy < seconds or reps < 2:
        oc.st = copy.deepcopy(st0)
        t0 = time.time()
        _, _, imp = oc.decode(wl.queries(w, reps)[:n_seq], 1 / math.sqrt(128), imp0.copy(), w.decay)
        oc.evict(imp, keep_k, w.q_window, w.recent_window)
        busy += time.time() - t0
        reps += 1
    hc = host_cpu(n_seq * w.Hkv)
    return {"value": n_seq * reps / busy, "unit": "tokens/s", "cores": hc["threads"],
            "kind": "oracle", "nproc": hc["nproc"], "cpu_model": hc["model"],
            "sample": f"{n_seq} of {w.B} sequences at full length, {reps} decode+evict steps "
                      f"in {busy:.1f}s (fp64 C, decode OpenMP over (sequence, kv head) pairs, "
                      f"eviction over sequences)"}


def evict_bench(args, w):
    """Timed step = decode with importance accumulation + windowed top-k
    evict with table compaction, from the same cache state every step (the
    cache metadata and the importance are restored outside the timed
    region; eviction never moves KV bytes).  Step time is GPU time (HIP
    events around the two calls)."""
    import torch

    from eviction_kvq_decode_amd import workloads as wl

    total_steps = args.warmup + args.steps
    t0 = time.time()
    n = wl.seq_lengths(w)
    n_cap = int(n.max()) + w.extra_steps + w.append_steps
    toks = wl.lockstep_tokens(w, n_cap, threads=min(16, os.cpu_count() or 1))
    g = wl.geometry_for(w, toks.seq_tags)
    log(f"[gen] {w.name}: tokens generated in {time.time() - t0:.1f}s; geometry {g}")
    t0 = time.time()
    cache = build_gpu_cache(w, toks, g)
    log(f"[gpu] cache built in {time.time() - t0:.1f}s")
    valid = toks.keep[:, : toks.tags.shape[0]].T & (toks.tags != wl.TAG_SKIP)
    kvb = kv_bytes(toks.tags[valid], w.Hkv)
    n_valid = int(valid.sum())
    B = w.B
    meta = {k: v.clone() for k, v in cache.t.items() if not k.startswith("kv")}
    IMP0 = torch.from_numpy(np.stack([wl.importance0(w, b, g.n_cap) for b in range(B)])).cuda()
    IMP = IMP0.clone()
    KK = torch.from_numpy(wl.keep_counts(w)).cuda()
    Q = torch.from_numpy(np.stack([wl.queries(w, s) for s in range(total_steps)])).cuda()
    out = torch.empty((B, w.Hq, 128), device="cuda")
    mass = torch.empty((B, g.n_cap), device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(total_steps)]
    for s in range(total_steps):
        for k, v in meta.items():
            cache.t[k].copy_(v)
        IMP.copy_(IMP0)
        ev[s][0].record()
        cache.decode(Q[s], out, mass, IMP, w.decay)
        ev[s][1].record()
        cache.evict(IMP, KK, w.q_window, w.recent_window)
        ev[s][2].record()
    torch.cuda.synchronize()
    if cache.status != 0:
        raise RuntimeError(f"status {cache.status} after timed steps")
    dec_ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(args.warmup, total_steps)])
    evi_ms = np.array([ev[s][1].elapsed_time(ev[s][2]) for s in range(args.warmup, total_steps)])
    # eviction: importance and position of every valid slot read once, the
    # table rewritten (4 B per entry), masks of the blocks touched (2 B)
    evb = n_valid * 8 + int(cache.t["n_blocks"].sum().item()) * 6
    # segment-granular eviction on the same state and importance, timed alone
    # (outside the step: an alternative to the top-k call, not a third stage)
    tbe_ms = []
    for s in range(total_steps):
        for k, v in meta.items():
            cache.t[k].copy_(v)
        IMP.copy_(IMP0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.evict_tbe(IMP, *TBE_PARAMS, w.q_window, w.recent_window)
        e1.record()
        tbe_ms.append((e0, e1))
    torch.cuda.synchronize()
    if cache.status != 0:
        raise RuntimeError(f"status {cache.status} after segment eviction")
    tbe_ms = np.array([a.elapsed_time(b) for a, b in tbe_ms[args.warmup:]])
    tbe_kept = valid_slot_count(cache)
    tam_ms = []
    for s in range(total_steps):
        for k, v in meta.items():
            cache.t[k].copy_(v)
        IMP.copy_(IMP0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cache.evict_tam(IMP, KK, *TAM_PARAMS, w.q_window, w.recent_window)
        e1.record()
        tam_ms.append((e0, e1))
    torch.cuda.synchronize()
    if cache.status != 0:
        raise RuntimeError(f"status {cache.status} after budgeted eviction")
    tam_ms = np.array([a.elapsed_time(b) for a, b in tam_ms[args.warmup:]])
    tam_kept = valid_slot_count(cache)
    step_ms = dec_ms + evi_ms
    achieved = kvb / (dec_ms.mean() * 1e-3) / 1e9
    ev_gbs = evb / (evi_ms.mean() * 1e-3) / 1e9
    log(f"[gpu] step {step_ms.mean() * 1e3:.1f} us: decode {dec_ms.mean() * 1e3:.1f} us "
        f"({achieved:.0f} GB/s of {kvb / 1e6:.1f} MB), evict {evi_ms.mean() * 1e3:.1f} us; "
        f"segment eviction {tbe_ms.mean() * 1e3:.1f} us, {n_valid} -> {tbe_kept} valid slots; "
        f"segment budgets {tam_ms.mean() * 1e3:.1f} us, {n_valid} -> {tam_kept}")
    result = {
        "metric": METRIC,
        "value": B / (step_ms.mean() * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": float(step_ms.mean()),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B} Hq={w.Hq} Hkv={w.Hkv} D=128, "
                               f"{int(n.min())}-{int(n.max())} positions/seq; step = decode with "
                               f"importance (decay {w.decay}) + top-k evict and compaction, "
                               f"from the same cache state each step",
                   "global_batch": B, "seq_len": int(n.max()),
                   "compressed_kv_mb_per_step": round(kvb / 1e6, 1)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": committed_traffic(args.workload),
                     "kernel": DECODE_KERNEL, "avg_us": float(dec_ms.mean() * 1e3),
                     "us": {"mean": float(dec_ms.mean() * 1e3), "p10": float(np.quantile(dec_ms, 0.1) * 1e3),
                            "p50": float(np.median(dec_ms) * 1e3), "p90": float(np.quantile(dec_ms, 0.9) * 1e3)}},
        "evict": {"kernel": "kvq_evict_topk (keys + select, compact and push)", "avg_us": float(evi_ms.mean() * 1e3),
                  "bytes": evb, "achieved_gbs": ev_gbs, "frac": ev_gbs / HBM_PEAK_GBS},
        "evict_tbe": {"kernel": "kvq_evict_tbe (prep + drop + compact and push)", "avg_us": float(tbe_ms.mean() * 1e3),
                      "r0_rmin_tkeep": list(TBE_PARAMS), "valid_before": n_valid,
                      "valid_after": tbe_kept, "bytes": evb,
                      "achieved_gbs": evb / (tbe_ms.mean() * 1e-3) / 1e9},
        "evict_tam": {"kernel": "kvq_evict_tam (prep + drop + compact and push)",
                      "avg_us": float(tam_ms.mean() * 1e3), "pivot_c_min_seg": list(TAM_PARAMS),
                      "valid_before": n_valid, "valid_after": tam_kept, "bytes": evb,
                      "achieved_gbs": evb / (tam_ms.mean() * 1e-3) / 1e9},
        "cpu_baseline": None,
    }
    del Q
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline_evict(w, toks, min(2, B), args.cpu_seconds)
    print(json.dumps(result), flush=True)


def ct_bench(args, w):
    """Continuous-thinking loop: every step appends one token per sequence
    and decodes (importance accumulated), and every `period` steps the cache
    is pruned to the budget (ct_loop.ContinuousThinking).  The first --warmup
    steps are untimed; all remaining steps of the generation are timed, each
    with HIP events around its calls.  Reports per-step GPU time (the time
    per output token of one layer), the prune steps apart, and the cache
    footprint: table blocks and valid tokens before and after the loop."""
    import torch

    from eviction_kvq_decode_amd import workloads as wl
    from eviction_kvq_decode_amd.ct_loop import ContinuousThinking

    t0 = time.time()
    n0 = int(wl.seq_lengths(w).max())
    toks = wl.lockstep_tokens(w, n0 + w.extra_steps, threads=min(16, os.cpu_count() or 1))
    g = wl.geometry_for(w, toks.seq_tags)
    log(f"[gen] {w.name}: tokens generated in {time.time() - t0:.1f}s; geometry {g}")
    cache = build_gpu_cache(w, toks, g)
    del toks
    tags_all = wl.loop_tags(w, n0 + w.loop_steps)
    steps = [wl.loop_step_tokens(w, s, tags_all) for s in range(w.loop_steps)]
    K = torch.from_numpy(np.stack([x[0] for x in steps])).cuda()
    V = torch.from_numpy(np.stack([x[1] for x in steps])).cuda()
    tags_host = np.stack([x[2] for x in steps])
    T = torch.from_numpy(tags_host).cuda()
    Q = torch.from_numpy(np.stack([wl.queries(w, s) for s in range(64)])).cuda()
    del steps
    B = w.B
    out = torch.empty((B, w.Hq, 128), device="cuda")
    mass = torch.empty((B, g.n_cap), device="cuda")
    st0 = cache.state_numpy()
    last_tags = tags_all[np.arange(w.B), n0 - 1]
    ct = ContinuousThinking(cache, w.keep, w.period, w.q_window, w.recent_window, w.decay,
                            policy=args.policy, tbe=TBE_PARAMS, tam=CT_TAM_PARAMS, last_tags=last_tags)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(w.loop_steps)]
    pruned = np.zeros(w.loop_steps, dtype=bool)
    torch.cuda.synchronize()
    for s in range(w.loop_steps):
        ev[s][0].record()
        pruned[s] = ct.step(K[s], V[s], T[s], Q[s % 64], out, mass, tags_host=tags_host[s])
        ev[s][1].record()
    torch.cuda.synchronize()
    if cache.status != 0:
        raise RuntimeError(f"status {cache.status} after the loop")
    ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(w.loop_steps)])[args.warmup:]
    pr = pruned[args.warmup:]
    st1 = cache.state_numpy()

    def footprint(st):
        blocks = int(st["n_blocks"].sum())
        valid = sum(bin(int(m)).count("1") for p in range(3)
                    for m in st[f"mask{p}"][st[f"mask{p}"] != 0])
        return blocks, valid

    b0, v0 = footprint(st0)
    b1, v1 = footprint(st1)
    us = ms * 1e3
    log(f"[gpu] {len(us)} timed steps: {us.mean():.1f} us/step (p50 {np.median(us):.1f}, "
        f"p90 {np.quantile(us, 0.9):.1f}); prune steps {us[pr].mean():.1f} us, others "
        f"{us[~pr].mean():.1f} us; table blocks {b0} -> {b1}, valid tokens {v0} -> {v1}")
    result = {
        "metric": METRIC,
        "value": B / (ms.mean() * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": int(len(ms)),
        "warmup": args.warmup,
        "ms_per_step": float(ms.mean()),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B} Hq={w.Hq} Hkv={w.Hkv} D=128, {n0} cached tokens/seq, "
                               f"{w.loop_steps} generated; windows {w.q_window}/{w.recent_window}; "
                               + (f"pruned by segment where a Transition starts (tbe {TBE_PARAMS})"
                                  if args.policy == "tbe" else
                                  f"pruned to {w.keep} every {w.period} tokens ({args.policy}"
                                  + (f", window of {CT_TAM_PARAMS[2]} queries" if args.policy == "tam" else "")
                                  + ")")
                               + "; step = append + decode (+ evict)",
                   "global_batch": B, "seq_len": n0 + w.loop_steps},
        "roofline": None,
        "ct": {"policy": args.policy,
               "us_per_step_p50": float(np.median(us)), "us_per_step_p90": float(np.quantile(us, 0.9)),
               "us_prune_step": float(us[pr].mean()) if pr.any() else None,
               "us_other_step": float(us[~pr].mean()),
               "table_blocks_before": b0, "table_blocks_after": b1,
               "valid_tokens_before": v0, "valid_tokens_after": v1,
               "tokens_appended": B * w.loop_steps,
               "slot_fill_after": v1 / (16.0 * b1) if b1 else None},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_evicted")
    ap.add_argument("--policy", choices=("topk", "tbe", "tam"), default="topk",
                    help="pruning of the continuous-thinking loop (--workload ct_loop)")
    ap.add_argument("--codec", choices=("int", "native"), default="int",
                    help="integer min/max codes, or ThinKV's E4M3 / E2M1 / ternary formats")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run 3 device-to-device copies of this many MiB before the steps "
                         "(a kernel of known traffic, to scale hardware byte counters)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/decode_long_evicted_traffic.json from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of runs with "
                         "--copy-probe-mb 1024, and exit (no GPU use)")
    args = ap.parse_args()
    if args.traffic_record:
        rec = traffic_record(*args.traffic_record, copy_mb=1024)
        with open(os.path.join(ROOT, "profiles", "decode_long_evicted_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the path shards by sequence "
                                   "with no exchange (see the design notes)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from eviction_kvq_decode_amd import kvq
    from eviction_kvq_decode_amd import workloads as wl

    kvq.lib()
    torch.cuda.set_device(0)
    w = wl.WORKLOADS[args.workload]
    if args.codec == "native":
        w = wl.scaled(w, codec=1)
    if w.period:
        ct_bench(args, w)
        return
    if w.keep or w.keep_frac:
        evict_bench(args, w)
        return
    total_steps = args.warmup + args.steps
    w = wl.scaled(w, extra_steps=max(w.extra_steps, total_steps + 8))
    t0 = time.time()
    n = wl.seq_lengths(w)
    n_cap = int(n.max()) + w.extra_steps + w.append_steps
    toks = wl.lockstep_tokens(w, n_cap, threads=min(16, os.cpu_count() or 1))
    g = wl.geometry_for(w, toks.seq_tags)
    log(f"[gen] {w.name}: tokens generated in {time.time() - t0:.1f}s; geometry {g}")
    # compressed-KV bytes the decode must read at each step
    valid = toks.keep[:, : toks.tags.shape[0]].T & (toks.tags != wl.TAG_SKIP)
    base_bytes = kv_bytes(toks.tags[valid], w.Hkv)
    # a cache that fits in the 256 MB Infinity Cache (MALL) would be served
    # from it on the next step: rotate copies whose total exceeds it twice over
    n_copies = max(1, math.ceil(MALL_ROTATE_BYTES / base_bytes))
    t0 = time.time()
    caches = [build_gpu_cache(w, toks, g) for _ in range(n_copies)]
    log(f"[gpu] {n_copies} cache cop{'y' if n_copies == 1 else 'ies'} built in {time.time() - t0:.1f}s")
    B = w.B
    steps_k, steps_v, steps_t, steps_q, step_bytes = [], [], [], [], []
    acc = [base_bytes] * n_copies
    for s in range(total_steps):
        k, v, tags = wl.step_tokens(w, s)
        steps_k.append(k), steps_v.append(v), steps_t.append(tags)
        steps_q.append(wl.queries(w, s))
        acc[s % n_copies] += kv_bytes(tags, w.Hkv)
        step_bytes.append(acc[s % n_copies])
    K = torch.from_numpy(np.stack(steps_k)).cuda()
    V = torch.from_numpy(np.stack(steps_v)).cuda()
    T = torch.from_numpy(np.stack(steps_t)).cuda()
    Q = torch.from_numpy(np.stack(steps_q)).cuda()
    out = torch.empty((B, w.Hq, 128), device="cuda")
    mass = torch.empty((B, g.n_cap), device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(total_steps)]

    def step(s):
        cache = caches[s % n_copies]
        cache.append(K[s], V[s], T[s])
        ev[s][0].record()
        cache.decode(Q[s], out, mass)
        ev[s][1].record()

    if args.copy_probe_mb > 0:
        src = torch.ones(args.copy_probe_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[gpu] copy probe: 3 x {args.copy_probe_mb} MB read + written")
        del src, dst
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, total_steps):
        step(s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    for cache in caches:
        if cache.status != 0:
            raise RuntimeError(f"status {cache.status} after timed steps")
    dec_ms = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(args.warmup, total_steps)])
    dec_bytes = step_bytes[args.warmup:]
    achieved = sum(dec_bytes) / (dec_ms.sum() * 1e-3) / 1e9
    ms_per_step = dt * 1e3 / args.steps
    dec_us = {"mean": float(dec_ms.mean() * 1e3), "p10": float(np.quantile(dec_ms, 0.1) * 1e3),
              "p50": float(np.median(dec_ms) * 1e3), "p90": float(np.quantile(dec_ms, 0.9) * 1e3)}
    log(f"[gpu] step {ms_per_step * 1e3:.1f} us, decode call {dec_us['mean']:.1f} us "
        f"(p10 {dec_us['p10']:.1f}, p50 {dec_us['p50']:.1f}, p90 {dec_us['p90']:.1f}), "
        f"{dec_bytes[-1] / 1e6:.1f} MB compressed KV, {achieved:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": B * args.steps / dt,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B} Hq={w.Hq} Hkv={w.Hkv} D=128, "
                               f"{int(n.max())} logical positions/seq, "
                               f"{100 * (1 - toks.keep[:, : int(n.max())].mean()):.0f}% evicted, "
                               + ("R/E/T as E4M3/E2M1/ternary" if w.codec else "R/E/T at 8/4/2 bits")
                               + "; step = append 1 token/seq + decode",
                   "global_batch": B, "seq_len": int(n.max()),
                   "compressed_kv_mb_per_step": round(dec_bytes[-1] / 1e6, 1)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": committed_traffic(args.workload) if not w.codec else None,
                     "kernel": DECODE_KERNEL, "avg_us": dec_us["mean"], "us": dec_us,
                     "cache_copies": n_copies},
        "cpu_baseline": None,
    }
    del K, V, Q
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, toks, min(args.cpu_seqs, B), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
