"""Continuous-thinking decode loop over the library's calls.

Pages (cited by title and section):
  - "ThinKV: Thought-Adaptive KV Cache Compression for Efficient Reasoning
    Models", Methodology, System Implementation (Continuous Thinking): a new
    token of a thought type overwrites an evicted slot of a block of that
    type in place, so a long generation under a cache budget keeps reusing
    the same blocks instead of compacting them.
  - "Dynamic Thinking-Token Selection ...", section 2.3: the question and
    recent windows are kept, top-k by accumulated importance among the rest
    (policy "topk", pruned every P new tokens).
  - "ThinKV", Methodology, think-before-evict (policy "tbe"): the eviction
    fires when a Transition thought is detected, in the sequences where it
    was, with kvq_evict_tbe's annealed retention by segment.
  - "Thought-Aware KV Cache Compaction ... (TAM)", section 2 (policy "tam"):
    segment budgets and pivotal tokens from the attention mass the last R
    queries gave each position (the selection window, 2.B), compacting every
    P new tokens (2.D).

One step appends one token per sequence and decodes (output and per-position
mass).  Policies "topk" and "tbe" accumulate the mass into the importance
with the decay (H2O-style); "tam" accumulates it, with no decay, into a
window score over the R decodes that end at each prune (the first of them
starts it afresh).  All work is enqueued on one stream; nothing here
computes or synchronises.
"""
from __future__ import annotations

import numpy as np

from . import kvq

TAG_T = kvq.TAG_T


class ContinuousThinking:
    """A decode loop with eviction on one cache."""

    POLICIES = ("topk", "tbe", "tam")

    def __init__(self, cache: kvq.Cache, budget: int, period: int, q_window: int = 0,
                 recent_window: int = 0, decay: float = 0.9, importance=None, policy: str = "topk",
                 tbe=(64, 4, 8), tam=(8.0, 16, 64), last_tags=None):
        """tbe = (r0, r_min, t_keep) for policy "tbe"; tam = (pivot_c,
        min_seg, window) for policy "tam", window = R <= period queries.
        last_tags: the thought type of each sequence's last cached token
        (host, [B]), so that a Transition continuing from the cache is not
        taken for a new one; None: no sequence ends in a Transition."""
        import torch

        if period < 1 or budget < 0:
            raise ValueError("period must be >= 1 and budget >= 0")
        if policy not in self.POLICIES:
            raise ValueError(f"policy must be one of {self.POLICIES}")
        self.policy, self.tbe = policy, tuple(tbe)
        self.pivot_c, self.min_seg, self.window = float(tam[0]), int(tam[1]), int(tam[2])
        if policy == "tam" and not 1 <= self.window <= period:
            raise ValueError("the TAM selection window must hold 1 .. period queries")
        g = cache.g
        self.cache, self.period, self.decay = cache, period, decay
        self.q_window, self.recent_window = q_window, recent_window
        dev = cache.device
        self.importance = importance if importance is not None else torch.zeros(
            (g.B, g.n_cap), dtype=torch.float32, device=dev)
        # TAM's window score: mass from the last R queries before a prune
        self.window_score = torch.zeros((g.B, g.n_cap), dtype=torch.float32, device=dev) \
            if policy == "tam" else None
        self.keep = torch.full((g.B,), budget, dtype=torch.int32, device=dev)
        self.prev_tags = (np.full(g.B, 255, dtype=np.uint8) if last_tags is None
                          else np.asarray(last_tags, dtype=np.uint8).copy())
        self.since_evict = 0

    def transition_onsets(self, tags_host) -> np.ndarray:
        """uint8 [B]: 1 where this step's token starts a Transition thought."""
        t = np.asarray(tags_host, dtype=np.uint8)
        return ((t == TAG_T) & (self.prev_tags != TAG_T)).astype(np.uint8)

    def step(self, k_new, v_new, tags, q, out, mass, stream=None, tags_host=None) -> bool:
        """Append, decode, and evict as the policy says; returns whether this
        step evicted.  tags_host: this step's tags on the host (the thought
        classifier's output), needed by policy "tbe" to see Transitions
        start."""
        import torch

        self.cache.append(k_new, v_new, tags, stream)
        self.since_evict += 1
        if self.policy == "tam":
            # window decodes: the R ending at the prune; the first restarts it
            first = self.period - self.window + 1
            if self.since_evict >= first:
                self.cache.decode(q, out, mass, self.window_score, 0.0 if self.since_evict == first else 1.0,
                                  stream=stream)
            else:
                self.cache.decode(q, out, mass, None, stream=stream)
        else:
            self.cache.decode(q, out, mass, self.importance, self.decay, stream=stream)

        if self.policy == "tbe":
            if tags_host is None:
                raise ValueError('policy "tbe" needs the host-side tags of each step')
            onset = self.transition_onsets(tags_host)
            self.prev_tags = np.asarray(tags_host, dtype=np.uint8).copy()
            if not onset.any():
                return False
            mask = torch.from_numpy(onset).to(self.cache.device)
            self.cache.evict_tbe(self.importance, *self.tbe, self.q_window, self.recent_window, stream,
                                 seq_mask=mask)
            self.last_onset = onset
            return True
        if self.since_evict < self.period:
            return False
        if self.policy == "tam":
            self.cache.evict_tam(self.window_score, self.keep, self.pivot_c, self.min_seg, self.q_window,
                                 self.recent_window, stream)
        else:
            self.cache.evict(self.importance, self.keep, self.q_window, self.recent_window, stream)
        self.since_evict = 0
        return True
