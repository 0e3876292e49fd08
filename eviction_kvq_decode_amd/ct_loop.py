"""Continuous-thinking decode loop over the library's three calls.

Pages (cited by title and section):
  - "ThinKV: Thought-Adaptive KV Cache Compression for Efficient Reasoning
    Models", Methodology, System Implementation (Continuous Thinking): a new
    token of a thought type overwrites an evicted slot of a block of that
    type in place, so a long generation under a cache budget keeps reusing
    the same blocks instead of compacting them.
  - "Thought-Aware KV Cache Compaction ... (TAM)", section 2.D (periodic
    compaction): pruning runs every P new tokens, so the cache size moves
    between the budget t and t + P.
  - "Dynamic Thinking-Token Selection ...", section 2.3: the question and
    recent windows are kept, top-k by accumulated importance among the rest.
  - "ThinKV", Methodology, think-before-evict: the loop can prune by thought
    segment instead (policy "tbe": kvq_evict_tbe's annealed retention).
  - "TAM", section 2: or by segment budgets with pivotal tokens (policy
    "tam": kvq_evict_tam, the accumulated importance as the window score).

One step appends one token per sequence, decodes (output and per-position
mass, accumulated into the importance with the decay), and every `period`
steps prunes the cache outside the windows: to `budget` tokens (top-k or
TAM budgets) or by the TBE schedule.  All work is enqueued on one stream;
nothing here computes or synchronises.
"""
from __future__ import annotations

from . import kvq


class ContinuousThinking:
    """A decode loop with periodic windowed top-k eviction on one cache."""

    POLICIES = ("topk", "tbe", "tam")

    def __init__(self, cache: kvq.Cache, budget: int, period: int, q_window: int = 0,
                 recent_window: int = 0, decay: float = 0.9, importance=None, policy: str = "topk",
                 tbe=(64, 4, 8), tam=(8.0, 16)):
        """tbe = (r0, r_min, t_keep) for policy "tbe"; tam = (pivot_c,
        min_seg) for policy "tam"."""
        import torch

        if period < 1 or budget < 0:
            raise ValueError("period must be >= 1 and budget >= 0")
        if policy not in self.POLICIES:
            raise ValueError(f"policy must be one of {self.POLICIES}")
        self.policy, self.tbe, self.tam = policy, tuple(tbe), tuple(tam)
        g = cache.g
        self.cache, self.period, self.decay = cache, period, decay
        self.q_window, self.recent_window = q_window, recent_window
        self.importance = importance if importance is not None else torch.zeros(
            (g.B, g.n_cap), dtype=torch.float32, device=cache.device)
        self.keep = torch.full((g.B,), budget, dtype=torch.int32, device=cache.device)
        self.since_evict = 0

    def step(self, k_new, v_new, tags, q, out, mass, stream=None) -> bool:
        """Append, decode, and evict if `period` tokens have arrived since the
        last eviction; returns whether this step evicted."""
        self.cache.append(k_new, v_new, tags, stream)
        self.cache.decode(q, out, mass, self.importance, self.decay, stream=stream)
        self.since_evict += 1
        if self.since_evict < self.period:
            return False
        if self.policy == "tbe":
            self.cache.evict_tbe(self.importance, *self.tbe, self.q_window, self.recent_window, stream)
        elif self.policy == "tam":
            self.cache.evict_tam(self.importance, self.keep, *self.tam, self.q_window, self.recent_window,
                                 stream)
        else:
            self.cache.evict(self.importance, self.keep, self.q_window, self.recent_window, stream)
        self.since_evict = 0
        return True
