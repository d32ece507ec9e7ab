"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random tensors with fixed shapes and distributions.  It
holds none of the speculative-decoding arithmetic (no norm, no attention, no
softmax, no sampling rule) and imports nothing else from this package, so both
the HIP path and the CPU oracle can be fed from it without sharing code.

Every tensor has its own torch generator, seeded from a CRC of
``(seed, model tag, layer, tensor name)``, so a tensor's values do not depend
on which other tensors were drawn first.  Values are drawn in float32 and
rounded to bfloat16 by torch (round-to-nearest-even) when the model is bf16.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Decoder shape: a Qwen-style dense pre-norm decoder (RMSNorm, RoPE, SwiGLU)."""
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    dtype: str            # "bf16" or "f32"
    tied: bool = False    # LM head shares the embedding table
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    mtp: bool = False     # carries one extra multi-token-prediction layer

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def layer_params(self) -> int:
        d, q, kv, f = self.d_model, self.q_dim, self.kv_dim, self.d_ffn
        return d * q + 2 * d * kv + q * d + 3 * d * f

    def streamed_params(self) -> int:
        """Parameters a forward streams (all layers + LM head; embedding rows are gathered)."""
        return self.n_layers * self.layer_params() + self.vocab * self.d_model

    def mtp_params(self) -> int:
        return 2 * self.d_model * self.d_model + self.layer_params()

    def with_layers(self, n_layers: int) -> "ModelShape":
        return dataclasses.replace(self, n_layers=n_layers, name=f"{self.name}-L{n_layers}")


# Shapes of the workloads.  The tiny pair is the fp32 correctness pair; the others
# are bf16 shapes of the Qwen family sizes the workloads name.
SHAPES: Dict[str, ModelShape] = {
    "tiny_target": ModelShape("tiny_target", 2, 128, 4, 4, 32, 512, 256, "f32"),
    "tiny_draft": ModelShape("tiny_draft", 1, 64, 2, 2, 32, 256, 256, "f32"),
    "qwen8b": ModelShape("qwen8b", 36, 4096, 32, 8, 128, 12288, 151936, "bf16"),
    "qwen0p6b": ModelShape("qwen0p6b", 28, 1024, 16, 8, 128, 3072, 151936, "bf16", tied=True),
    "qwen27b": ModelShape("qwen27b", 64, 5120, 40, 8, 128, 17408, 151936, "bf16"),
    "qwen0p8b": ModelShape("qwen0p8b", 24, 1024, 8, 4, 128, 3584, 151936, "bf16", tied=True),
    "qwen9b_mtp": ModelShape("qwen9b_mtp", 32, 4096, 32, 8, 128, 12288, 151936, "bf16", mtp=True),
}

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd")


def tensor_seed(seed: int, tag: str, layer: int, name: str) -> int:
    return zlib.crc32(f"{seed}:{tag}:{layer}:{name}".encode()) & 0x7FFFFFFF


def _torch_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def _normal(shape, std: float, s: int, device: str, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(s)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


# RMSNorm gains are drawn per tensor from N(1, GAIN_STD^2), so that every gain multiply and the
# choice of gain at each norm matter to the results.
GAIN_STD = 0.1


def _gain(n: int, s: int, device: str, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(s)
    x = torch.randn((n,), generator=g, device=device, dtype=torch.float32)
    return x.mul_(GAIN_STD).add_(1.0).to(dtype)


def layer_shapes(shape: ModelShape) -> Dict[str, tuple]:
    d, q, kv, f = shape.d_model, shape.q_dim, shape.kv_dim, shape.d_ffn
    return {
        "attn_norm": (d,), "wq": (q, d), "wk": (kv, d), "wv": (kv, d), "wo": (d, q),
        "ffn_norm": (d,), "wg": (f, d), "wu": (f, d), "wd": (d, f),
    }


def make_layer(shape: ModelShape, seed: int, tag: str, layer: int, device: str = "cpu",
               std: float = 0.02) -> Dict[str, torch.Tensor]:
    dt = _torch_dtype(shape.dtype)
    out = {}
    for name, shp in layer_shapes(shape).items():
        if name.endswith("norm"):
            out[name] = _gain(shp[0], tensor_seed(seed, tag, layer, name), device, dt)
        else:
            out[name] = _normal(shp, std, tensor_seed(seed, tag, layer, name), device, dt)
    return out


def make_weights(shape: ModelShape, seed: int = 0, device: str = "cpu", tag: Optional[str] = None,
                 std: float = 0.02) -> Dict[str, object]:
    """Random-init N(0, std) weights, RMSNorm gains N(1, GAIN_STD^2), nn.Linear layout [out, in].

    Returns {"embed", "lm_head", "final_norm", "layers": [dict per layer], "mtp": dict|None}.
    With ``shape.tied`` the LM head is the embedding tensor itself (no copy).
    """
    tag = tag or shape.name
    dt = _torch_dtype(shape.dtype)
    V, d = shape.vocab, shape.d_model
    embed = _normal((V, d), std, tensor_seed(seed, tag, -1, "embed"), device, dt)
    lm_head = embed if shape.tied else _normal((V, d), std, tensor_seed(seed, tag, -1, "lm_head"),
                                               device, dt)
    w = {
        "embed": embed,
        "lm_head": lm_head,
        "final_norm": _gain(d, tensor_seed(seed, tag, -1, "final_norm"), device, dt),
        "layers": [make_layer(shape, seed, tag, l, device, std) for l in range(shape.n_layers)],
        "mtp": None,
    }
    if shape.mtp:
        w["mtp"] = make_mtp(shape, seed, device, tag, std)
    return w


# fp8 weights are drawn as such: each weight is an E4M3 code times a per-row float32 scale.
# Codes are N(0, 1) values clipped to +-6.5, times FP8_UNIT, rounded to E4M3 by torch (so
# magnitudes reach 416 of the format's 448 and the subnormal codes occur); each row's scale is
# std / FP8_UNIT times U(0.75, 1.25), so rows differ and a weight is about N(0, std^2).
FP8_UNIT = 64.0
PROJ_TENSORS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def _fp8_codes(shape, s: int, device: str) -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(s)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    x.clamp_(-6.5, 6.5).mul_(FP8_UNIT)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def _row_scales(rows: int, std: float, s: int, device: str) -> torch.Tensor:
    g = torch.Generator(device=device).manual_seed(s)
    u = torch.rand((rows,), generator=g, device=device, dtype=torch.float32)
    return (u * 0.5 + 0.75) * (std / FP8_UNIT)


def make_weights_fp8(shape: ModelShape, seed: int = 0, device: str = "cpu", tag: Optional[str] = None,
                     std: float = 0.02) -> Dict[str, object]:
    """Like make_weights for a bf16 shape, with the seven projections of every layer and the
    LM head (untied) as uint8 E4M3 code tensors [out, in] plus "<name>_scale" float32 [out]
    row scales ("lm_head_scale" for the head).  Embedding and norm gains stay bf16."""
    if shape.dtype != "bf16" or shape.tied or shape.mtp:
        raise ValueError("fp8 weights: bf16 shapes with an untied LM head and no MTP layer")
    tag = (tag or shape.name) + ":fp8"
    V, d = shape.vocab, shape.d_model
    layers = []
    for l in range(shape.n_layers):
        lw = {}
        for name, shp in layer_shapes(shape).items():
            if name.endswith("norm"):
                lw[name] = _gain(shp[0], tensor_seed(seed, tag, l, name), device, torch.bfloat16)
            else:
                lw[name] = _fp8_codes(shp, tensor_seed(seed, tag, l, name), device)
                lw[name + "_scale"] = _row_scales(shp[0], std, tensor_seed(seed, tag, l, name + "_scale"), device)
        layers.append(lw)
    return {
        "embed": _normal((V, d), std, tensor_seed(seed, tag, -1, "embed"), device, torch.bfloat16),
        "lm_head": _fp8_codes((V, d), tensor_seed(seed, tag, -1, "lm_head"), device),
        "lm_head_scale": _row_scales(V, std, tensor_seed(seed, tag, -1, "lm_head_scale"), device),
        "final_norm": _gain(d, tensor_seed(seed, tag, -1, "final_norm"), device, torch.bfloat16),
        "layers": layers,
        "mtp": None,
    }


def make_gdn_inputs(T: int, n_heads: int, d_k: int, d_v: int, seed: int = 0, device: str = "cpu"):
    """Inputs of T tokens to one linear-attention layer and its committed state, float32:
    q [T, H, d_k] ~ N(0, 1/d_k); k [T, H, d_k] uniform on the unit sphere (normalized normal
    draws); v [T, H, d_v] ~ N(0, 1); decays alpha [T, H] ~ U(0.8, 1); write strengths
    beta [T, H] ~ U(0.1, 0.9); state [H, d_v, d_k] ~ N(0, 0.3^2)."""
    g = torch.Generator(device="cpu").manual_seed(tensor_seed(seed, "gdn", T, f"{n_heads}:{d_k}:{d_v}"))
    q = torch.randn((T, n_heads, d_k), generator=g) / d_k ** 0.5
    k = torch.randn((T, n_heads, d_k), generator=g)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((T, n_heads, d_v), generator=g)
    alpha = torch.rand((T, n_heads), generator=g) * 0.2 + 0.8
    beta = torch.rand((T, n_heads), generator=g) * 0.8 + 0.1
    state = torch.randn((n_heads, d_v, d_k), generator=g) * 0.3
    return {n: t.to(device=device, dtype=torch.float32).contiguous()
            for n, t in dict(q=q, k=k, v=v, alpha=alpha, beta=beta, state=state).items()}


def make_mtp(shape: ModelShape, seed: int, device: str, tag: str, std: float = 0.02):
    """One extra decoder layer plus its input norms and the [d, 2d] input projection."""
    dt = _torch_dtype(shape.dtype)
    d = shape.d_model
    m = make_layer(shape, seed, tag + ":mtp", 0, device, std)
    for name in ("norm_h", "norm_e", "final_norm"):
        m[name] = _gain(d, tensor_seed(seed, tag + ":mtp", 0, name), device, dt)
    m["w_proj"] = _normal((d, 2 * d), std, tensor_seed(seed, tag + ":mtp", 0, "w_proj"), device, dt)
    return m


def make_kv_prefix(shape: ModelShape, length: int, seed: int = 0, device: str = "cpu",
                   tag: Optional[str] = None, n_layers: Optional[int] = None):
    """Synthetic cached keys/values for ``length`` earlier positions, N(0, 1).

    Returns (K, V), each [n_layers, n_kv_heads, length, head_dim] in the model dtype.
    Keys are taken as already position-rotated (that is how a cache stores them).
    """
    tag = tag or shape.name
    nl = shape.n_layers if n_layers is None else n_layers
    dt = _torch_dtype(shape.dtype)
    shp = (nl, shape.n_kv_heads, length, shape.head_dim)
    k = _normal(shp, 1.0, tensor_seed(seed, tag, -2, "kv_k"), device, dt)
    v = _normal(shp, 1.0, tensor_seed(seed, tag, -2, "kv_v"), device, dt)
    return k, v


def make_tokens(n: int, vocab: int, seed: int, tag: str = "prompt") -> np.ndarray:
    """n uniform token ids in [0, vocab), int32."""
    rng = np.random.default_rng(tensor_seed(seed, tag, -3, "tokens"))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def make_accept_logits(batch: int, k: int, vocab: int, sigma: float, seed: int = 0,
                       device: str = "cpu", copies: int = 1):
    """Logits for the stand-alone truncation/accept workload.

    target: [copies, batch, k+1, vocab] bf16 ~ N(0, 3)
    draft:  [copies, batch, k,   vocab] bf16 = target[..., :k, :] + N(0, sigma)
    Draft row j predicts the same position as target row j.
    """
    g = torch.Generator(device=device).manual_seed(tensor_seed(seed, f"acc:{batch}:{k}:{sigma}", -4, "t"))
    t = torch.randn((copies, batch, k + 1, vocab), generator=g, device=device, dtype=torch.float32)
    t.mul_(3.0)
    g2 = torch.Generator(device=device).manual_seed(tensor_seed(seed, f"acc:{batch}:{k}:{sigma}", -4, "d"))
    noise = torch.randn((copies, batch, k, vocab), generator=g2, device=device, dtype=torch.float32)
    d = t[:, :, :k, :] + noise.mul_(sigma)
    return t.to(torch.bfloat16), d.to(torch.bfloat16)


def make_copy_stream(n: int, vocab: int, seed: int = 0, copy_frac: float = 0.4,
                     span_lo: int = 32, span_hi: int = 256) -> np.ndarray:
    """Copy-heavy token stream: segments of U[span_lo, span_hi] tokens, each either a copy of a
    random earlier window or fresh uniform tokens, chosen to keep the copied fraction near
    ``copy_frac``.  The first segment is uniform.  Returns int32 [n]."""
    rng = np.random.default_rng(tensor_seed(seed, "copy_stream", -5, f"{n}:{vocab}"))
    out: List[int] = []
    copied = 0
    while len(out) < n:
        span = int(rng.integers(span_lo, span_hi + 1))
        want_copy = len(out) >= span_lo and (copied / max(len(out), 1)) < copy_frac
        if want_copy:
            span = min(span, len(out))
            start = int(rng.integers(0, len(out) - span + 1))
            seg = out[start:start + span]
            copied += len(seg)
        else:
            seg = rng.integers(0, vocab, size=span).tolist()
        out.extend(int(t) for t in seg)
    return np.asarray(out[:n], dtype=np.int32)


def to_numpy_f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a (bf16 or f32) tensor, on the host."""
    return t.detach().to("cpu", torch.float32).numpy()


def weights_to_numpy(w: Dict[str, object]) -> Dict[str, object]:
    """Host float32 copies (exact for bf16 values) of a weight dict, for the oracle."""
    def cv(x):
        return None if x is None else to_numpy_f32(x)
    out = {
        "embed": cv(w["embed"]),
        "final_norm": cv(w["final_norm"]),
        "layers": [{k: cv(v) for k, v in lw.items()} for lw in w["layers"]],
        "mtp": None if w.get("mtp") is None else {k: cv(v) for k, v in w["mtp"].items()},
    }
    out["lm_head"] = out["embed"] if w["lm_head"] is w["embed"] else cv(w["lm_head"])
    return out


def weights_to(w: Dict[str, object], device: str) -> Dict[str, object]:
    """Copy a weight dict to ``device``, keeping a tied LM head tied (one tensor)."""
    def mv(x):
        return None if x is None else x.to(device)
    out = {
        "embed": mv(w["embed"]),
        "final_norm": mv(w["final_norm"]),
        "layers": [{k: mv(v) for k, v in lw.items()} for lw in w["layers"]],
        "mtp": None if w.get("mtp") is None else {k: mv(v) for k, v in w["mtp"].items()},
    }
    out["lm_head"] = out["embed"] if w["lm_head"] is w["embed"] else mv(w["lm_head"])
    return out
