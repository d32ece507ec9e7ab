"""Truncation, sampling and the accept rule (oracle side), all decisions in float32.

Passages followed:

* "Qwen3.5 and Qwen3.6 MTP head reaches 1.4x on Apple Silicon after three fixes",
  section "The verify was wrong under sampling": accept a drafted token with
  probability min(1, p_main/q_draft); on rejection draw the replacement from the
  clipped, rescaled difference of the two distributions, i.e. normalize(max(0, p - q)).
  Greedy verification compares the draft with the main model's argmax.
* Same page, "Truncation has to match on both sides": the draft and the verify side
  both apply the same top_k / top_p truncation (top 20 tokens, top 0.95 of the mass).
* "Speculative decoding on Apple Silicon" (OptiQ docs), "MTP head": the sampler is
  temperature, top_p and top_k.
* "What is Speculative Decoding and How Does a Draft Model Work?", "#2": drafted tokens up
  to the first disagreement are kept and the target's own token replaces the first
  disagreeing one, so one target pass yields at least one token; "#3": at temperature 0
  a draft is kept only when it is exactly the target's most likely token.

Readings where the pages are silent (each is listed in the design notes):

* order of truncation: divide by temperature, keep the top_k largest (ties: lower id
  first), softmax over the kept set (max-subtracted), walk in that order keeping a token
  while the exclusive running sum is below top_p (the first is always kept), renormalize;
* all running sums are sequential float32 sums in a stated order;
* temperature 0 means greedy: a one-hot list at the argmax (lowest id on ties);
* sampling walks the list in ascending id order and returns the first id whose running
  sum exceeds u * Z (Z = the list's sequential sum), else the last id with mass;
* a draft is accepted iff u < p(d) / q(d) (float32 IEEE division, strict compare);
* when every draft is accepted a bonus token is drawn from the last target row;
* a residual with zero mass falls back to sampling from p.

Near-tie margins: a discrete outcome decided by a float comparison is reported with its
margin so that a caller can tell a real disagreement from a rounding-order one.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

F32 = np.float32
NEAR_TIE = 1e-6


@dataclasses.dataclass
class TokenList:
    """A truncated distribution: ids ascending, float32 probabilities (sum ~1)."""
    ids: np.ndarray      # int64, ascending
    probs: np.ndarray    # float32
    margin: float = np.inf      # top_p boundary: |exclusive running sum - top_p| (prob units)
    gap_logit: float = np.inf   # argmax gap (greedy) or k-th minus (k+1)-th scaled logit

    def prob(self, tok: int) -> np.float32:
        i = np.searchsorted(self.ids, tok)
        if i < len(self.ids) and self.ids[i] == tok:
            return self.probs[i]
        return F32(0.0)

    def argmax(self) -> int:
        # largest probability, lowest id on ties (ids are ascending)
        return int(self.ids[int(np.argmax(self.probs))])


def seq_sum(x: np.ndarray) -> np.float32:
    """Sequential float32 sum in array order (np.cumsum accumulates left to right)."""
    x = np.asarray(x, dtype=F32)
    if x.size == 0:
        return F32(0.0)
    return np.cumsum(x, dtype=F32)[-1]


def seq_cumsum(x: np.ndarray) -> np.ndarray:
    return np.cumsum(np.asarray(x, dtype=F32), dtype=F32)


def order_desc(z: np.ndarray) -> np.ndarray:
    """Indices sorted by (-z, id): largest value first, lower id first among equals."""
    ids = np.arange(z.shape[0])
    return np.lexsort((ids, -z.astype(np.float64)))


def scaled_logits(logits: np.ndarray, temperature: float) -> np.ndarray:
    z = np.asarray(logits, dtype=F32)
    if np.any(np.isnan(z)) or np.any(np.isposinf(z)):
        raise ValueError("logits hold NaN or +inf")
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        z = (z / F32(temperature)).astype(F32)
    return z + F32(0.0)      # -0.0 becomes +0.0, so equal values tie on id only


def truncate(logits: np.ndarray, temperature: float, top_k: int, top_p: float) -> TokenList:
    """One row of logits -> the truncated distribution the sampler draws from."""
    z0 = np.asarray(logits, dtype=F32)
    if np.any(np.isnan(z0)) or np.any(np.isposinf(z0)):
        raise ValueError("logits hold NaN or +inf")
    if not np.any(np.isfinite(z0)):
        raise ValueError("no finite logit: empty support")
    if temperature <= 0.0:
        # greedy: argmax, lowest id on ties
        order = order_desc(z0 + F32(0.0))
        a = int(order[0])
        gap = np.inf
        if len(order) > 1 and np.isfinite(z0[order[1]]):
            gap = float(np.float64(z0[a]) - np.float64(z0[order[1]]))
        return TokenList(np.array([a], dtype=np.int64), np.array([1.0], dtype=F32), np.inf, gap)

    z = scaled_logits(z0, temperature)
    V = z.shape[0]
    order = order_desc(z)
    kk = V if (top_k <= 0 or top_k >= V) else int(top_k)
    gap = np.inf
    if kk < V and np.isfinite(z[order[kk]]):
        gap = float(np.float64(z[order[kk - 1]]) - np.float64(z[order[kk]]))
    kept = order[:kk]
    kept = kept[np.isfinite(z[kept])]
    zk = z[kept]
    m = zk[0]
    with np.errstate(over="ignore", under="ignore"):
        e = np.exp((zk - m).astype(F32)).astype(F32)
    S = seq_sum(e)
    p = (e / S).astype(F32)
    margin = np.inf
    n_keep = len(p)
    tp = F32(top_p)
    if top_p < 1.0:
        c = seq_cumsum(p)
        excl = np.concatenate([[F32(0.0)], c[:-1]]).astype(F32)
        keep = excl < tp
        keep[0] = True
        n_keep = int(np.count_nonzero(keep))   # keep is a prefix: excl is nondecreasing
        # margin of the boundary decisions: last kept and first dropped
        cand = [abs(float(excl[n_keep - 1]) - float(tp))] if n_keep > 1 else []
        if n_keep < len(p):
            cand.append(abs(float(excl[n_keep]) - float(tp)))
        if cand:
            margin = min(cand)
    p = p[:n_keep]
    ids = kept[:n_keep]
    Z = seq_sum(p)
    p = (p / Z).astype(F32)
    srt = np.argsort(ids, kind="stable")
    return TokenList(ids[srt].astype(np.int64), p[srt], margin, gap)


def sample(ids: np.ndarray, weights: np.ndarray, u: np.float32) -> Tuple[int, float]:
    """Inverse-CDF draw in ascending id order from unnormalized float32 weights.

    Returns (token, margin): the first id whose running sum c exceeds u * Z, or the last
    id with nonzero weight if rounding leaves none; margin = |c - u*Z| at the deciding
    step(s)."""
    w = np.asarray(weights, dtype=F32)
    Z = seq_sum(w)
    t = F32(F32(u) * Z)
    c = seq_cumsum(w)
    hit = np.nonzero(c > t)[0]
    if len(hit):
        i = int(hit[0])
    else:
        nz = np.nonzero(w > 0)[0]
        i = int(nz[-1]) if len(nz) else len(w) - 1
    margin = abs(float(c[i]) - float(t))
    if i > 0:
        margin = min(margin, abs(float(c[i - 1]) - float(t)))
    return int(ids[i]), margin


@dataclasses.dataclass
class AcceptResult:
    n: int                     # accepted drafts, 0..K
    tokens: List[int]          # n+1 emitted tokens: accepted drafts, then correction/bonus
    margin: float              # smallest decision margin met (|u - p/q| or a CDF step)


def residual(p: TokenList, q: TokenList) -> np.ndarray:
    """max(0, p - q) over p's support (ascending ids), float32."""
    qv = np.array([q.prob(int(t)) for t in p.ids], dtype=F32)
    return np.maximum(F32(0.0), (p.probs - qv).astype(F32)).astype(F32)


def accept(drafts: Sequence[int], q: Sequence[TokenList], p: Sequence[TokenList], greedy: bool,
           u_acc: Optional[Sequence[np.float32]] = None,
           u_res: Optional[np.float32] = None) -> AcceptResult:
    """The accept rule for one sequence: K drafts, K draft lists q_1..q_K and K+1 target
    lists p_0..p_K (p_{j-1} scores the position drafted by d_j)."""
    K = len(drafts)
    assert len(p) == K + 1 and len(q) == K
    out: List[int] = []
    margin = np.inf
    for j in range(K):
        d = int(drafts[j])
        if greedy:
            a = p[j].argmax()
            if d == a:
                out.append(d)
                continue
            out.append(a)
            return AcceptResult(j, out, margin)
        pj = p[j].prob(d)
        qj = q[j].prob(d)
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = F32(F32(pj) / F32(qj))
        u = F32(u_acc[j])
        if np.isfinite(ratio):
            margin = min(margin, abs(float(u) - float(ratio)))
        if u < ratio:
            out.append(d)
            continue
        r = residual(p[j], q[j])
        if seq_sum(r) > 0:
            tok, m2 = sample(p[j].ids, r, u_res)
        else:
            tok, m2 = sample(p[j].ids, p[j].probs, u_res)
        out.append(tok)
        return AcceptResult(j, out, min(margin, m2))
    # every draft accepted: bonus token from the last target row
    if greedy:
        out.append(p[K].argmax())
        return AcceptResult(K, out, margin)
    tok, m2 = sample(p[K].ids, p[K].probs, u_res)
    out.append(tok)
    return AcceptResult(K, out, min(margin, m2))
