"""An independent batched decoder built from torch's own CPU operators (``rms_norm``,
``scaled_dot_product_attention`` with an explicit causal mask, ``silu``), float64 between the
bf16 contract's rounding points.  It computes all positions at once, where the oracle loops
over single-token forwards, and shares no code with the oracle: the pins compare the two.

The layer is the plain pre-norm decoder the workload shapes describe (RMSNorm, rotate-half
RoPE, grouped-query attention, SwiGLU); with ``bf16`` the normed rows, q, k, v, the
attention output and the SwiGLU product are rounded to bfloat16 and the residual stream to
float32."""
import numpy as np
import torch
import torch.nn.functional as F


def _w(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _rb(t, bf16):
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64) if bf16 else t


def _rf(t, bf16):
    return t.to(torch.float32).to(torch.float64) if bf16 else t


def torch_layers(spec, layers, x, P=0, k_prefix=None, v_prefix=None, bf16=False):
    """Decoder layers over the M rows x [M, d] (float64 tensor) at positions P .. P+M-1, each
    attending the cached prefix (k_prefix / v_prefix [n_layers, n_kv, P, hd]) and the rows up
    to itself.  Returns the residual rows after the last layer."""
    M = x.shape[0]
    T = P + M
    hd, nq, nkv = spec.head_dim, spec.n_q_heads, spec.n_kv_heads
    pos = torch.arange(P, T, dtype=torch.float64)
    inv = spec.rope_theta ** (-2.0 * torch.arange(hd // 2, dtype=torch.float64) / hd)
    ang = pos[:, None] * inv[None, :]
    cos, sin = torch.cos(ang), torch.sin(ang)

    def rot(t):  # t [M, heads, hd]
        a, b = t[..., : hd // 2], t[..., hd // 2:]
        c, s = cos[:, None, :], sin[:, None, :]
        return torch.cat([a * c - b * s, b * c + a * s], dim=-1)

    rb = lambda t: _rb(t, bf16)
    rf = lambda t: _rf(t, bf16)
    mask = torch.ones(M, T, dtype=torch.bool).tril(diagonal=P)
    for l, lw in enumerate(layers):
        n1 = rb(F.rms_norm(x, (spec.d_model,), _w(lw["attn_norm"]), eps=spec.rms_eps))
        q = rb(rot((n1 @ _w(lw["wq"]).T).view(M, nq, hd)))
        k = rb(rot((n1 @ _w(lw["wk"]).T).view(M, nkv, hd)))
        v = rb((n1 @ _w(lw["wv"]).T).view(M, nkv, hd))
        kk, vv = k.transpose(0, 1), v.transpose(0, 1)
        if P:
            kk = torch.cat([_w(k_prefix[l]), kk], dim=1)
            vv = torch.cat([_w(v_prefix[l]), vv], dim=1)
        kk = kk.repeat_interleave(nq // nkv, dim=0)
        vv = vv.repeat_interleave(nq // nkv, dim=0)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), kk, vv, attn_mask=mask)
        o = rb(o.transpose(0, 1).reshape(M, nq * hd))
        x = rf(x + o @ _w(lw["wo"]).T)
        n2 = rb(F.rms_norm(x, (spec.d_model,), _w(lw["ffn_norm"]), eps=spec.rms_eps))
        h = rb(F.silu(n2 @ _w(lw["wg"]).T) * (n2 @ _w(lw["wu"]).T))
        x = rf(x + h @ _w(lw["wd"]).T)
    return x


def torch_head(spec, final_norm, lm_head, x, bf16=False):
    """Final RMSNorm and vocabulary projection of residual rows x: float32 logits."""
    xf = _rb(F.rms_norm(x, (spec.d_model,), _w(final_norm), eps=spec.rms_eps), bf16)
    return (xf @ _w(lm_head).T).to(torch.float32).numpy()


def torch_forward(spec, W, tokens, k_prefix=None, v_prefix=None, bf16=False):
    """Batched causal forward over all positions at once."""
    P = 0 if k_prefix is None else k_prefix.shape[2]
    x = _w(W["embed"])[torch.as_tensor(np.asarray(tokens), dtype=torch.long)]
    x = torch_layers(spec, W["layers"], x, P, k_prefix, v_prefix, bf16)
    return torch_head(spec, W["final_norm"], W["lm_head"], x, bf16)


def torch_mtp(spec, W, h_prev, tokens, P=0, k_prefix=None, v_prefix=None, bf16=False):
    """Multi-token-prediction head over rows i = 0..M-1 at positions P + i, each fed the
    hidden row h_prev[i] and the token tokens[i]: the two inputs RMS-normalized with their own
    gains and concatenated as [hidden part; token part], projected by w_proj [d, 2d], one
    decoder layer with its own cache, the head's final RMSNorm and the shared LM head.
    Returns (logits [M, V] float32, hidden rows [M, d])."""
    m = W["mtp"]
    rb = lambda t: _rb(t, bf16)
    a = rb(F.rms_norm(_w(h_prev), (spec.d_model,), _w(m["norm_h"]), eps=spec.rms_eps))
    e = _w(W["embed"])[torch.as_tensor(np.asarray(tokens), dtype=torch.long)]
    b = rb(F.rms_norm(e, (spec.d_model,), _w(m["norm_e"]), eps=spec.rms_eps))
    x = _rf(torch.cat([a, b], dim=1) @ _w(m["w_proj"]).T, bf16)
    x = torch_layers(spec, [m], x, P, k_prefix, v_prefix, bf16)
    return torch_head(spec, m["final_norm"], W["lm_head"], x, bf16), x.numpy()
