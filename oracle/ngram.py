"""N-gram lookup drafting and the acceptance-rate gate (oracle side).

"Speculative decoding on Apple Silicon" (OptiQ docs), "N-gram lookup: any model": when
the last few tokens match something earlier in the context, draft the tokens that
followed that earlier occurrence and verify them in one pass; ``--ngram-min`` is the
shortest match that triggers a draft (default 3) and ``--ngram-draft N`` the most tokens
drafted per step (8 recommended).  The draft length is not fixed: one verification pass
is timed when the model loads, and each step's length is chosen from how often recent
drafts were accepted (``--no-ngram-gate`` always drafts N when a match exists).

Readings (the pages give no formula):

* match: among earlier end positions e (e <= n-2), the match length ell(e) is the number of
  tokens, up to ``max_match``, for which ctx[e-i] == ctx[n-1-i]; take the largest ell >=
  ``n_min`` and, among equals, the most recent e; draft ctx[e+1 : e+1+k], never past the
  end of the context;
* gate: alpha = exponential moving average of accepted/attempted over recent steps
  (weight 0.5, starting at 1); c(k) = t_verify(k) / t_verify(0) from the load-time timings;
  choose k in 0..N maximizing (sum_{i=0..k} alpha^i) / (c(k) + k * t_draft / t_verify(0)),
  the expected tokens per step over the step's cost.  k = 0 means no draft this step.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def match_lengths(ctx: Sequence[int], max_match: int) -> np.ndarray:
    """ell(e) for every earlier end position e in 0..n-2 (brute force, pure Python)."""
    n = len(ctx)
    out = np.zeros(max(n - 1, 0), dtype=np.int64)
    for e in range(n - 1):
        ell = 0
        while ell < max_match and e - ell >= 0 and ctx[e - ell] == ctx[n - 1 - ell]:
            ell += 1
        out[e] = ell
    return out


def ngram_draft(ctx: Sequence[int], k: int, n_min: int = 3, max_match: int = 16):
    """Returns (drafts list of <= k tokens, match length, end position e or -1)."""
    n = len(ctx)
    if n < 2 or k <= 0:
        return [], 0, -1
    ell = match_lengths(ctx, max_match)
    best = int(ell.max()) if len(ell) else 0
    if best < n_min:
        return [], 0, -1
    e = int(np.nonzero(ell == best)[0][-1])     # most recent among the longest
    drafts = [int(t) for t in ctx[e + 1: min(e + 1 + k, n)]]
    return drafts, best, e


class Gate:
    """Acceptance-rate gate choosing the per-step draft length."""

    def __init__(self, n_max: int, verify_cost: Sequence[float], draft_cost: float = 0.0,
                 enabled: bool = True, weight: float = 0.5):
        assert len(verify_cost) >= n_max + 1
        self.n_max = n_max
        self.c = [float(t) / float(verify_cost[0]) for t in verify_cost[: n_max + 1]]
        self.td = float(draft_cost) / float(verify_cost[0])
        self.enabled = enabled
        self.w = weight
        self.alpha = 1.0

    def choose(self) -> int:
        if not self.enabled:
            return self.n_max
        best_k, best_v = 0, -1.0
        for k in range(self.n_max + 1):
            gain = sum(self.alpha ** i for i in range(k + 1))
            v = gain / (self.c[k] + k * self.td)
            if v > best_v + 1e-12:
                best_k, best_v = k, v
        return best_k

    def update(self, accepted: int, attempted: int):
        if attempted > 0:
            self.alpha = self.w * self.alpha + (1.0 - self.w) * (accepted / attempted)
