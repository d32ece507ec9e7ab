"""Linear-attention layer state and its speculative rollback (oracle side; test
infrastructure, imported only by tests, the smoke check and the benchmark's CPU baseline).

"Speculative Decoding on Apple Silicon: 119% Faster...", section "Why this needed a patch to
mlx_lm at all": hybrid models mix full-attention layers with Gated DeltaNet-style linear
attention layers.  A full-attention layer rolls back by dropping the rejected entries of its
key/value list; a linear-attention layer has folded every token it saw into one fixed-size
recurrent state, so rollback keeps a snapshot of the state from before the speculative
forward and, once the accepted prefix is known, restores it and runs only the accepted tokens
through the recurrence again.  The same page, "What this means in practice", puts the cost of
that replay window in memory.

The pages do not write the recurrence down.  The reading taken here is the gated delta rule
of the Gated DeltaNet layer (Yang, Kautz and Hatamizadeh, "Gated Delta Networks: Improving
Mamba2 with Delta Rule"), per head, with a state S of d_v rows and d_k columns:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    o_t = S_t q_t

with the decay alpha_t and the write strength beta_t in (0, 1) and q_t, k_t as the layer's
projections leave them (the normalization of q and k and the gate activations belong to those
projections and are inputs here).  Arithmetic is float64, written in the matrix form above.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def step(S: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: float, beta: float) -> np.ndarray:
    """One token of the gated delta rule for one head: S [d_v, d_k] -> the next state."""
    S = np.asarray(S, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_k = k.shape[0]
    transition = np.eye(d_k) - beta * np.outer(k, k)
    return alpha * (S @ transition) + beta * np.outer(v, k)


def run(S0: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray,
        beta: np.ndarray) -> Tuple[np.ndarray, List[np.ndarray]]:
    """Tokens t = 0 .. T-1 through every head from the states S0 [H, d_v, d_k].

    q, k [T, H, d_k]; v [T, H, d_v]; alpha, beta [T, H].  Returns the outputs o [T, H, d_v]
    (o_t from the state after token t) and the states after each token (T arrays [H, d_v, d_k]).
    """
    S = np.array(S0, dtype=np.float64)
    T, H = alpha.shape
    out = np.zeros((T, H, v.shape[2]))
    states = []
    for t in range(T):
        for h in range(H):
            S[h] = step(S[h], k[t, h], v[t, h], float(alpha[t, h]), float(beta[t, h]))
            out[t, h] = S[h] @ np.asarray(q[t, h], dtype=np.float64)
        states.append(S.copy())
    return out, states


def speculate(S0: np.ndarray, q, k, v, alpha, beta, n_keep: int):
    """The pages' mechanism: snapshot the committed state, run all T speculative tokens,
    then restore the snapshot and replay only the first n_keep of them.  In a verify over
    [last token, d_1 .. d_K] that accepts n drafts, n_keep = n + 1 (the last token and the
    accepted drafts; the token the verify emits is the next cycle's first input).  Returns
    (outputs of the T tokens, the committed state after the n_keep kept tokens)."""
    if not 0 <= n_keep <= alpha.shape[0]:
        raise ValueError("n_keep out of range")
    snapshot = np.array(S0, dtype=np.float64)
    out, _ = run(snapshot, q, k, v, alpha, beta)
    S = snapshot.copy()  # restore
    for t in range(n_keep):
        for h in range(S.shape[0]):
            S[h] = step(S[h], k[t, h], v[t, h], float(alpha[t, h]), float(beta[t, h]))
    return out, S
