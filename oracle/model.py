"""Decoder forward, one token at a time (oracle side).

What the pages fix and what is a reading:

* "What is Speculative Decoding and How Does a Draft Model Work?", "#2": the target checks
  all drafted tokens in one pass, the same way it reads a prompt.  A pass over K+1
  positions therefore yields, at each position, exactly the logits a sequence of K+1
  single-token forwards would yield.  The oracle computes it that way (``forward_tokens``
  loops over tokens), so it needs no block-causal mask and cannot depend on K.
* "Speculative Decoding on Apple Silicon: 119% Faster...", "Why this needed a patch to
  mlx_lm at all": a plain attention layer keeps a per-token key/value list that is rolled
  back by slicing rejected entries off the end (``KVCache.trim``).
* Same page, "The original result: Qwen3-8B and a 0.6B draft": the 8B target has ordinary
  attention layers throughout.

The layer itself is a reading (the pages give no formula): the Qwen-style dense pre-norm
decoder that the workload shapes describe.  x = E[t]; per layer
x += Wo . Attn(RoPE(Wq n1), RoPE(Wk n1), Wv n1) with n1 = RMSNorm(x), then
x += Wd . (silu(Wg n2) * (Wu n2)) with n2 = RMSNorm(x); logits = Wlm . RMSNorm(x).
RMSNorm eps 1e-6, rotate-half RoPE with theta 1e6, no biases, q-head h reads kv-head
floor(h * n_kv / n_q), scale 1/sqrt(head_dim).

Arithmetic is float64.  For a bf16 model the precision contract rounds to bfloat16 the
normed rows RMSNorm(x) * g that the projections read, q, k and v (k and v are stored that
way), the attention output and the SwiGLU product, and keeps the residual stream in float32;
softmax weights and logits are float32 quantities (computed in float64 here).  An f32 model
rounds nothing but the final logits to float32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

from .numerics import round_bf16, round_f32


@dataclasses.dataclass(frozen=True)
class Spec:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    bf16: bool
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    # float32 arithmetic between the rounding points instead of float64: the same contract
    # evaluated the way a float32 implementation would, to measure how far two correct
    # evaluations of it drift apart (its bf16 rounding points amplify float32 rounding)
    arith32: bool = False

    @staticmethod
    def from_shape(s, arith32: bool = False) -> "Spec":
        return Spec(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.d_ffn,
                    s.vocab, s.dtype == "bf16", s.rms_eps, s.rope_theta, arith32)

    @property
    def dt(self):
        return np.float32 if self.arith32 else np.float64


class KVCache:
    """Per layer K and V: [n_kv_heads, capacity, head_dim] float64, plus a length."""

    def __init__(self, spec: Spec, capacity: int, n_layers: Optional[int] = None):
        nl = spec.n_layers if n_layers is None else n_layers
        self.k = [np.zeros((spec.n_kv_heads, capacity, spec.head_dim)) for _ in range(nl)]
        self.v = [np.zeros((spec.n_kv_heads, capacity, spec.head_dim)) for _ in range(nl)]
        self.length = 0

    def load_prefix(self, k: np.ndarray, v: np.ndarray):
        """k, v: [n_layers, n_kv, L, head_dim]."""
        L = k.shape[2]
        for l in range(len(self.k)):
            self.k[l][:, :L] = k[l]
            self.v[l][:, :L] = v[l]
        self.length = L

    def trim(self, new_length: int):
        """Roll back to the first ``new_length`` entries (slice off the end)."""
        if new_length > self.length:
            raise ValueError("trim beyond the current length")
        for l in range(len(self.k)):
            self.k[l][:, new_length:] = 0.0
            self.v[l][:, new_length:] = 0.0
        self.length = new_length


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float, dt=np.float64) -> np.ndarray:
    x = np.asarray(x, dtype=dt)
    return x / np.sqrt(np.mean(x * x) + dt(eps)) * np.asarray(g, dtype=dt)


def rope(x: np.ndarray, pos: int, theta: float, dt=np.float64) -> np.ndarray:
    """Rotate-half RoPE on [n_heads, head_dim]: pair i with i + head_dim/2, angle
    pos * theta^(-2i/head_dim)."""
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / hd)
    c, s = np.cos(ang).astype(dt), np.sin(ang).astype(dt)
    x = np.asarray(x, dtype=dt)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_kv: int, dt=np.float64) -> np.ndarray:
    """One query position: q [n_q, hd]; k, v [n_kv, T, hd] (every visible key) -> [n_q, hd]."""
    q, k, v = (np.asarray(a, dtype=dt) for a in (q, k, v))
    n_q, hd = q.shape
    out = np.empty_like(q)
    for h in range(n_q):
        kv = (h * n_kv) // n_q
        s = k[kv] @ q[h] / dt(np.sqrt(hd))
        s = s - s.max()
        w = np.exp(s)
        w = w / w.sum()
        out[h] = w @ v[kv]
    return out


def _w(a, dt=np.float64) -> np.ndarray:
    return np.asarray(a, dtype=dt)


def decoder_layer(spec: Spec, lw: Dict[str, np.ndarray], x: np.ndarray, pos: int,
                  kv: KVCache, l: int, trace: Optional[Dict] = None) -> np.ndarray:
    """One layer for one token at ``pos``; appends this position's k, v to layer l.  With
    ``trace`` (a dict) the layer's intermediate rows are recorded in it under their names."""
    dt = spec.dt
    bf = round_bf16 if spec.bf16 else (lambda a: a)
    rs = round_f32 if spec.bf16 and not spec.arith32 else (lambda a: a)
    hd = spec.head_dim
    x = np.asarray(x, dtype=dt)
    n1 = bf(rmsnorm(x, lw["attn_norm"], spec.rms_eps, dt))
    q_raw = _w(lw["wq"], dt) @ n1
    k_raw = _w(lw["wk"], dt) @ n1
    v = bf(_w(lw["wv"], dt) @ n1).reshape(spec.n_kv_heads, hd)
    q = bf(rope(q_raw.reshape(spec.n_q_heads, hd), pos, spec.rope_theta, dt))
    k = bf(rope(k_raw.reshape(spec.n_kv_heads, hd), pos, spec.rope_theta, dt))
    kv.k[l][:, pos] = k
    kv.v[l][:, pos] = v
    o = attend(q, kv.k[l][:, :pos + 1], kv.v[l][:, :pos + 1], spec.n_kv_heads, dt)
    o = bf(o.reshape(-1))
    x_mid = rs(x + _w(lw["wo"], dt) @ o)
    n2 = bf(rmsnorm(x_mid, lw["ffn_norm"], spec.rms_eps, dt))
    g = _w(lw["wg"], dt) @ n2
    u = _w(lw["wu"], dt) @ n2
    h = bf(silu(g) * u)
    x_out = rs(x_mid + _w(lw["wd"], dt) @ h)
    if trace is not None:
        trace.update(n1=n1, q_raw=q_raw, k_raw=k_raw, k=k.reshape(-1), v=v.reshape(-1), o=o,
                     x_mid=x_mid, n2=n2, h=h, x_out=x_out)
    return x_out


def forward_one(spec: Spec, W: Dict, kv: KVCache, pos: int, token: int, trace: Optional[List] = None):
    """Single-token forward at ``pos``.  Returns (logits float32 [V], hidden float64 [d]) where
    hidden is the last layer's residual output (before the final norm).  With ``trace`` (a
    list) one dict of intermediate rows per layer is appended to it."""
    x = _w(W["embed"][token], spec.dt)
    for l in range(spec.n_layers):
        tr = None if trace is None else {}
        x = decoder_layer(spec, W["layers"][l], x, pos, kv, l, tr)
        if trace is not None:
            trace.append(tr)
    bf = round_bf16 if spec.bf16 else (lambda a: a)
    xf = bf(rmsnorm(x, W["final_norm"], spec.rms_eps, spec.dt))
    logits = (_w(W["lm_head"], spec.dt) @ xf).astype(np.float32)
    return logits, x


def forward_tokens(spec: Spec, W: Dict, kv: KVCache, tokens, traces: Optional[List] = None) -> np.ndarray:
    """Forward over ``tokens`` at positions kv.length, kv.length+1, ...: a plain loop of
    single-token forwards.  Appends their k, v; returns float32 logits [M, V].  With
    ``traces`` (a list) each token's per-layer intermediates (a list of dicts) are appended."""
    out = []
    for t in tokens:
        pos = kv.length
        tr = None if traces is None else []
        logits, _ = forward_one(spec, W, kv, pos, int(t), tr)
        if traces is not None:
            traces.append(tr)
        kv.length = pos + 1
        out.append(logits)
    return np.stack(out)


def forward_tokens_hidden(spec: Spec, W: Dict, kv: KVCache, tokens):
    """As ``forward_tokens`` but also returns the hidden states [M, d]."""
    outs, hs = [], []
    for t in tokens:
        pos = kv.length
        logits, h = forward_one(spec, W, kv, pos, int(t))
        kv.length = pos + 1
        outs.append(logits)
        hs.append(h)
    return np.stack(outs), np.stack(hs)


# --- multi-token-prediction head (a reading; numerics "parity unpinned") ------------------
#
# "What is Speculative Decoding and How Does a Draft Model Work?", "MTP and the other
# drafting methods": a model trained for multi-token prediction carries a small set of extra
# layers that predict the following tokens as a by-product of the current one.  "Speculative
# decoding on Apple Silicon" (OptiQ docs), "Serving and the Lab": the head is a projection
# followed by a final layer.  Reading: input = concat(RMSNorm(h_t), RMSNorm(E[x_{t+1}])),
# projected [2d -> d], one decoder layer with its own cache at position t+1, a final
# RMSNorm and the target's own LM head (the head borrows the loaded weights: "Qwen3.5 and
# Qwen3.6 MTP head reaches 1.4x...", "Duplicate weights in unified memory").

def mtp_forward_one(spec: Spec, W: Dict, kv: KVCache, pos: int, h_prev: np.ndarray,
                    token: int):
    """One MTP step: (hidden at pos-1, token at pos) -> (logits [V] float32, hidden [d])."""
    M = W["mtp"]
    bf = round_bf16 if spec.bf16 else (lambda a: a)
    rs = round_f32 if spec.bf16 else (lambda a: a)
    a = bf(rmsnorm(h_prev, M["norm_h"], spec.rms_eps))
    b = bf(rmsnorm(_w(W["embed"][token]), M["norm_e"], spec.rms_eps))
    x = rs(_w(M["w_proj"]) @ np.concatenate([a, b]))
    x = decoder_layer(spec, M, x, pos, kv, 0)
    xf = bf(rmsnorm(x, M["final_norm"], spec.rms_eps))
    logits = (_w(W["lm_head"]) @ xf).astype(np.float32)
    return logits, x
