"""fp8 weight decoding (oracle side; test infrastructure, imported only by tests, the smoke
check and the benchmark's CPU baseline).

The pages run their models with quantized weights ("Speculative Decoding on Apple Silicon:
119% Faster...", section "Reproducing this"; "What is Speculative Decoding and How Does a
Draft Model Work?", section "The demo, draft model on and off with two pairings") but fix no
format.  The reading taken here: one byte per weight,
an E4M3 code of the OCP 8-bit floating point specification, and one float32 scale per output
row, weight[r][k] = value(code[r][k]) * scale[r].

E4M3 as that specification defines it: bit 7 sign s, bits 6..3 exponent e (bias 7), bits
2..0 mantissa m.  e = 0 is subnormal, (-1)^s * 2^-6 * m/8; otherwise (-1)^s * 2^(e-7) *
(1 + m/8), except e = 15 with m = 7, which is NaN (the format has no infinities, so the
largest finite magnitude is 2^8 * 1.75 = 448).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

PROJ = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def e4m3_value(code: int) -> float:
    """The value of one E4M3 code (0..255), from the bit fields."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError("code out of range")
    s = -1.0 if code >> 7 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * 2.0 ** -6 * (m / 8.0)
    return s * 2.0 ** (e - 7) * (1.0 + m / 8.0)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of E4M3 codes (uint8)."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("codes must be uint8")
    return E4M3_TABLE[codes]


def dequantize_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """weight[r][k] = value(code[r][k]) * scale[r], float64 [rows, in]."""
    scale = np.asarray(scale, dtype=np.float64)
    if codes.ndim != 2 or scale.shape != (codes.shape[0],):
        raise ValueError("one scale per row")
    return decode(codes) * scale[:, None]


def dequantize_model(w: Dict) -> Dict:
    """Oracle weight dict (float64 arrays) from an fp8 model given as numpy arrays: the seven
    projections of each layer and the LM head as uint8 codes with "<name>_scale" / "lm_head_scale"
    row scales; the embedding and norm gains as plain values."""
    out = {"embed": np.asarray(w["embed"], dtype=np.float64),
           "final_norm": np.asarray(w["final_norm"], dtype=np.float64),
           "lm_head": dequantize_rows(w["lm_head"], w["lm_head_scale"]), "layers": [], "mtp": None}
    for lw in w["layers"]:
        d = {"attn_norm": np.asarray(lw["attn_norm"], dtype=np.float64),
             "ffn_norm": np.asarray(lw["ffn_norm"], dtype=np.float64)}
        for n in PROJ:
            d[n] = dequantize_rows(lw[n], lw[n + "_scale"])
        out["layers"].append(d)
    return out
