"""The draft / verify / accept / trim loop and plain decoding (oracle side).

Passages followed:

* "Speculative Decoding on Apple Silicon: 119% Faster...", "How speculative decoding
  works": the draft proposes several tokens one at a time; the target checks them all in a
  single batched forward; the matching prefix is kept, the first mismatch is replaced by
  the target's own token, and the rest is discarded and regenerated next round.
* "What is Speculative Decoding and How Does a Draft Model Work?", "#1": plain decoding is
  one full target pass per token; "#2": one target pass always yields at least one token.
* "Speculative decoding on Apple Silicon" (OptiQ docs), "MTP head": acceptance is
  drafts_accepted / drafts_attempted.
* "Speculative Decoding on Apple Silicon: 119% Faster...", "Why this needed a patch to
  mlx_lm at all": the cache rolls back by slicing the rejected entries off its end.

Readings: the last accepted token t0 sits at position L (the cache holds 0..L-1); the
verify feeds [t0, d_1..d_K] at L..L+K; after n acceptances the target keeps L+1+n entries
and the emitted last token is the next cycle's t0.  The draft keeps min(its length,
L+1+n) entries and, before drafting, first feeds whatever history it has not consumed
(after a full acceptance that is d_K).  Prefill feeds the first P-1 prompt tokens; the
last prompt token is the first t0, so every generated token comes from ``accept`` and
K = 0 is plain decoding.  Uniforms: draft sample j -> counter (j, round, seq, 0); accept
test j -> (j, round, seq, 1); residual or bonus -> (0, round, seq, 2).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import philox
from .model import KVCache, Spec, forward_one, mtp_forward_one
from .ngram import Gate, ngram_draft
from .sampling import TokenList, accept, sample, truncate


@dataclasses.dataclass
class Sampler:
    temperature: float = 0.0
    top_k: int = 20
    top_p: float = 0.95

    @property
    def greedy(self) -> bool:
        return self.temperature <= 0.0


@dataclasses.dataclass
class CycleLog:
    L: int                      # target length before the verify (position of t0)
    drafts: List[int]
    n: int
    tokens: List[int]
    margin: float               # smallest accept/sampling margin in the cycle
    p_gap: List[float]          # per target row: logit gap of the argmax / top_k boundary
    q_gap: List[float]
    p_margin: List[float]       # per target row: top_p boundary margin
    q_margin: List[float]


@dataclasses.dataclass
class GenResult:
    tokens: List[int]
    cycles: List[CycleLog]
    drafts_attempted: int
    drafts_accepted: int


def draft_confidence(ql: TokenList, d: int) -> np.float32:
    """The draft model's confidence in its draft d: the probability its truncated list gives d
    (float32, as the list holds it).  Greedy lists are one-hot, so every greedy draft has
    confidence 1."""
    hit = ql.probs[ql.ids == d]
    return np.float32(hit[0]) if len(hit) else np.float32(0.0)


def keeps_drafting(ql: TokenList, d: int, p_min: float) -> bool:
    """The draft-probability control ("What is Speculative Decoding and How Does a Draft Model
    Work?", section "The demo, draft model on and off with two pairings": drafting stops once
    the draft model's confidence falls below the setting; 0 turns it off).  Reading: the draft
    whose confidence is below p_min is not proposed, and neither is any later one."""
    return not (p_min > 0.0) or bool(draft_confidence(ql, d) >= np.float32(p_min))


class DraftModel:
    """External draft model: its own weights and cache."""

    def __init__(self, spec: Spec, W: Dict, capacity: int):
        self.spec, self.W = spec, W
        self.kv = KVCache(spec, capacity)

    def propose(self, hist: List[int], L: int, K: int, sampler: Sampler, seed: int, rnd: int,
                seq: int = 0, p_min: float = 0.0):
        """Feed history up to position L (t0), then its own drafts: at most K, fewer when a
        draft's confidence falls below p_min (keeps_drafting)."""
        logits = None
        while self.kv.length <= L:
            pos = self.kv.length
            logits, _ = forward_one(self.spec, self.W, self.kv, pos, hist[pos])
            self.kv.length = pos + 1
        drafts, qs = [], []
        for j in range(1, K + 1):
            ql = truncate(logits, sampler.temperature, sampler.top_k, sampler.top_p)
            if sampler.greedy:
                d = ql.argmax()
            else:
                u = philox.uniform(seed, j, rnd, seq, philox.STREAM_DRAFT)
                d, _ = sample(ql.ids, ql.probs, u)
            if not keeps_drafting(ql, d, p_min):
                break
            drafts.append(d)
            qs.append(ql)
            if j < K:
                pos = self.kv.length
                logits, _ = forward_one(self.spec, self.W, self.kv, pos, d)
                self.kv.length = pos + 1
        return drafts, qs

    def trim(self, new_len: int):
        self.kv.trim(min(self.kv.length, new_len))


class MTPDraft:
    """Self-speculation through the target's MTP layer (a reading, see model.py)."""

    def __init__(self, spec: Spec, W: Dict, capacity: int, hidden: Dict[int, np.ndarray]):
        self.spec, self.W = spec, W
        self.kv = KVCache(spec, capacity, n_layers=1)
        self.hidden = hidden    # target hidden state by position (shared with the loop)

    def propose(self, hist, L, K, sampler, seed, rnd, seq=0, p_min=0.0):
        logits = h = None
        while self.kv.length <= L:
            pos = self.kv.length
            logits, h = mtp_forward_one(self.spec, self.W, self.kv, pos, self.hidden[pos - 1],
                                        hist[pos])
            self.kv.length = pos + 1
        drafts, qs = [], []
        for j in range(1, K + 1):
            ql = truncate(logits, sampler.temperature, sampler.top_k, sampler.top_p)
            if sampler.greedy:
                d = ql.argmax()
            else:
                u = philox.uniform(seed, j, rnd, seq, philox.STREAM_DRAFT)
                d, _ = sample(ql.ids, ql.probs, u)
            if not keeps_drafting(ql, d, p_min):
                break
            drafts.append(d)
            qs.append(ql)
            if j < K:
                pos = self.kv.length
                logits, h = mtp_forward_one(self.spec, self.W, self.kv, pos, h, d)
                self.kv.length = pos + 1
        return drafts, qs

    def trim(self, new_len: int):
        # the caller passes L+1: entries past position L were built from the head's own
        # hidden states rather than the target's, so they are dropped and rebuilt next cycle
        self.kv.trim(min(self.kv.length, new_len))


class AdaptiveDepth:
    """Adaptive draft length.  "Speculative decoding on Apple Silicon" (OptiQ docs), section
    "About depth" (and "Qwen3.5 and Qwen3.6 MTP head reaches 1.4x...", section "Why K=1 wins
    on Metal"): a heuristic that raises K after a cycle whose drafts were all accepted and
    lowers it after a cycle with a rejection.  The pages give no step sizes; the reading takes
    them as parameters (default one draft either way) and keeps K within [k_min, k_max].  A
    cycle that drafted nothing leaves K as it is."""

    def __init__(self, k0: int, k_min: int = 1, k_max: int = 8, up: int = 1, down: int = 1):
        assert 0 <= k_min <= k0 <= k_max and up >= 0 and down >= 0
        self.k, self.k_min, self.k_max, self.up, self.down = k0, k_min, k_max, up, down

    def choose(self) -> int:
        return self.k

    def update(self, accepted: int, attempted: int) -> None:
        assert 0 <= accepted <= attempted
        if attempted == 0:
            return
        if accepted == attempted:
            self.k = min(self.k_max, self.k + self.up)
        else:
            self.k = max(self.k_min, self.k - self.down)


def one_hot(tok: int) -> TokenList:
    return TokenList(np.array([tok], dtype=np.int64), np.array([1.0], dtype=np.float32))


def run(target_spec: Spec, target_W: Dict, tkv: KVCache, t0: int, hist: List[int], n_new: int,
        K: int, sampler: Sampler, seed: int, draft=None, ngram: Optional[Dict] = None,
        hidden: Optional[Dict[int, np.ndarray]] = None, seq: int = 0,
        teacher: Optional[Sequence[int]] = None, depth: Optional[AdaptiveDepth] = None,
        p_min: float = 0.0, min_draft: int = 0) -> GenResult:
    """Generate ``n_new`` tokens.  ``hist`` holds every token at positions < tkv.length plus
    t0 at position tkv.length.  ``draft`` is a DraftModel / MTPDraft or None; ``ngram`` a dict
    {n_min, max_match, gate: Gate|None}; ``teacher`` replaces the drafts by a known
    continuation: teacher[i] is the i-th generated token, so each cycle drafts the K entries
    after the tokens emitted so far.  ``depth`` (an AdaptiveDepth) picks each cycle's K for a
    draft model or teacher and is told every cycle's outcome.  ``p_min`` and ``min_draft`` are
    the draft controls of "What is Speculative Decoding and How Does a Draft Model Work?",
    section "The demo, draft model on and off with two pairings" (K is the most drafts): the
    draft model / MTP head stops at the first draft below the draft probability p_min
    (keeps_drafting), and a cycle with fewer drafts than min_draft (from a drafter, not a
    teacher) checks none of them, which makes it a plain decoding step."""
    assert len(hist) == tkv.length + 1 and hist[-1] == t0
    out: List[int] = []
    cycles: List[CycleLog] = []
    att = acc = 0
    rnd = 0
    while len(out) < n_new:
        L = tkv.length
        k = K = depth.choose() if depth is not None else K
        if ngram is not None:
            gate = ngram.get("gate")
            k = gate.choose() if gate is not None else K
            drafts, _, _ = ngram_draft(hist, k, ngram.get("n_min", 3), ngram.get("max_match", 16))
            qs = [one_hot(d) for d in drafts]
            k = len(drafts)
        elif teacher is not None:
            done = len(out)
            drafts = [int(t) for t in teacher[done: done + K]]
            k = len(drafts)
            qs = [one_hot(d) for d in drafts]
        elif draft is not None and K > 0:
            drafts, qs = draft.propose(hist, L, K, sampler, seed, rnd, seq, p_min)
        else:
            drafts, qs = [], []
        if teacher is None and len(drafts) < min_draft:
            drafts, qs = [], []
        k = len(drafts)
        # verify: one target pass over [t0, d_1..d_k] at positions L..L+k
        rows = [hist[L]] + drafts
        ps, gaps, pm = [], [], []
        for i, t in enumerate(rows):
            logits, h = forward_one(target_spec, target_W, tkv, L + i, t)
            tkv.length = L + i + 1
            if hidden is not None:
                hidden[L + i] = h
            pl = truncate(logits, sampler.temperature, sampler.top_k, sampler.top_p)
            ps.append(pl)
            gaps.append(pl.gap_logit)
            pm.append(pl.margin)
        if sampler.greedy:
            res = accept(drafts, qs, ps, True)
        else:
            u_acc = [philox.uniform(seed, j, rnd, seq, philox.STREAM_ACCEPT) for j in range(1, k + 1)]
            u_res = philox.uniform(seed, 0, rnd, seq, philox.STREAM_RESIDUAL)
            res = accept(drafts, qs, ps, False, u_acc, u_res)
        n = res.n
        # trim: keep t0 and the n accepted drafts
        tkv.trim(L + 1 + n)
        if draft is not None:
            draft.trim(L + 1 + n if not isinstance(draft, MTPDraft) else L + 1)
        # history: accepted drafts at L+1..L+n, then the correction / bonus at L+1+n,
        # which is the next cycle's t0
        hist.extend(int(t) for t in res.tokens)
        att += k
        acc += n
        if ngram is not None and ngram.get("gate") is not None:
            ngram["gate"].update(n, k)
        if depth is not None:
            depth.update(n, k)
        cycles.append(CycleLog(L, list(drafts), n, list(res.tokens), res.margin, gaps,
                               [ql.gap_logit for ql in qs], pm, [ql.margin for ql in qs]))
        out.extend(res.tokens)
        rnd += 1
    return GenResult(out[:n_new], cycles, att, acc)


def prefill(spec: Spec, W: Dict, kv: KVCache, tokens: Sequence[int]):
    """Feed tokens one by one; returns the hidden states by position."""
    hidden = {}
    for t in tokens:
        pos = kv.length
        _, h = forward_one(spec, W, kv, pos, int(t))
        kv.length = pos + 1
        hidden[pos] = h
    return hidden
