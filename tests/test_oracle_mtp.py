"""Pins for the oracle's multi-token-prediction head (``oracle.model.mtp_forward_one``).

The head is a reading of "What is Speculative Decoding and How Does a Draft Model Work?",
section "MTP and the other drafting methods" (extra layers that predict the following tokens
from the current one), and "Speculative decoding on Apple Silicon" (OptiQ docs), section
"Serving and the Lab" (a projection followed by a final layer): the hidden row at t-1 and the
embedding of the token at t, each RMS-normalized with its own gain, concatenated as
[hidden part; token part], projected [2d -> d], one decoder layer with its own cache, a final
RMSNorm and the target's LM head.

Checked here, without the GPU:
* against the independent batched torch implementation of ``tests.torch_ref`` (torch's
  ``rms_norm``, ``scaled_dot_product_attention``, ``silu``), float32 and bf16 models, with and
  without a cached prefix;
* closed forms: with all decoder-layer weights zero the layer is the identity (the attention
  values and the SwiGLU product are zero), so with w_proj = [0 | I] the logits are those of the
  normed token embedding alone and do not depend on the hidden row, and with w_proj = [I | 0]
  those of the normed hidden row alone and do not depend on the token.  A swapped concat order,
  a missing input norm or gain, or a missing final norm fails one of these.
"""
import numpy as np
import pytest

from oracle import numerics
from oracle.model import KVCache, Spec, mtp_forward_one
from speculative_decoding_token_amd import synth
from tests.torch_ref import torch_mtp

EPS = 1e-6


def mtp_model(dtype, seed=0, std=0.2):
    shape = synth.ModelShape("mtp_t", 1, 64, 4, 2, 16, 96, 50, dtype, mtp=True)
    W = synth.weights_to_numpy(synth.make_weights(shape, seed, std=std))
    return shape, Spec.from_shape(shape), W


def oracle_steps(spec, W, h_prev, tokens, P=0, kp=None, vp=None):
    kv = KVCache(spec, P + len(tokens) + 2, n_layers=1)
    if P:
        kv.load_prefix(kp, vp)
    out, hid = [], []
    for i, t in enumerate(tokens):
        lg, h = mtp_forward_one(spec, W, kv, P + i, h_prev[i], int(t))
        kv.length = P + i + 1
        out.append(lg)
        hid.append(h)
    return np.stack(out), np.stack(hid)


@pytest.mark.parametrize("dtype,P", [("f32", 0), ("f32", 7), ("bf16", 0), ("bf16", 9)])
def test_mtp_matches_batched_torch(dtype, P):
    shape, spec, W = mtp_model(dtype)
    rng = np.random.default_rng(5)
    M = 6
    h_prev = rng.normal(0, 1.5, (M, shape.d_model))
    if dtype == "bf16":
        h_prev = h_prev.astype(np.float32).astype(np.float64)  # the target's residual rows are float32
    tokens = synth.make_tokens(M, shape.vocab, 4)
    kp = vp = None
    if P:
        k, v = synth.make_kv_prefix(shape, P, 2, n_layers=1)
        kp, vp = synth.to_numpy_f32(k), synth.to_numpy_f32(v)
    got, hid = oracle_steps(spec, W, h_prev, tokens, P, kp, vp)
    ref, rhid = torch_mtp(spec, W, h_prev, tokens, P, kp, vp, bf16=(dtype == "bf16"))
    tol = 1e-6 if dtype == "bf16" else 1e-9
    assert np.abs(got - ref).max() / np.abs(ref).max() < tol
    assert np.abs(hid - rhid).max() / np.abs(rhid).max() < tol


def _zero_layer(W, first_half_identity: bool):
    m = dict(W["mtp"])
    for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
        m[name] = np.zeros_like(m[name])
    d = m["w_proj"].shape[0]
    eye, zero = np.eye(d), np.zeros((d, d))
    m["w_proj"] = np.concatenate([eye, zero] if first_half_identity else [zero, eye], axis=1)
    out = dict(W)
    out["mtp"] = m
    return out


def _normed(x, g, bf):
    x = np.asarray(x, np.float64)
    return bf(x / np.sqrt(np.mean(x * x) + EPS) * np.asarray(g, np.float64))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mtp_closed_forms_concat_order_and_norms(dtype):
    shape, spec, W = mtp_model(dtype, seed=3)
    bf = numerics.round_bf16 if dtype == "bf16" else (lambda a: a)
    rng = np.random.default_rng(9)
    h1 = rng.normal(0, 3.0, shape.d_model) * np.linspace(0.2, 2.0, shape.d_model)
    h2 = rng.normal(0, 0.1, shape.d_model)
    t1, t2 = 7, 31
    m = W["mtp"]
    lm = np.asarray(W["lm_head"], np.float64)

    def logits_of(Wz, h, t):
        kv = KVCache(spec, 4, n_layers=1)
        return mtp_forward_one(spec, Wz, kv, 0, h, t)[0].astype(np.float64)

    # token half only: x0 = normed embedding of the token
    Wt = _zero_layer(W, first_half_identity=False)
    a, b = logits_of(Wt, h1, t1), logits_of(Wt, h2, t1)
    assert np.array_equal(a, b)
    x0 = _normed(W["embed"][t1], m["norm_e"], bf)
    want = (lm @ _normed(x0, m["final_norm"], bf)).astype(np.float32)
    np.testing.assert_allclose(a, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
    assert not np.allclose(a, logits_of(Wt, h1, t2))
    # hidden half only: x0 = normed hidden row
    Wh = _zero_layer(W, first_half_identity=True)
    a, b = logits_of(Wh, h1, t1), logits_of(Wh, h1, t2)
    assert np.array_equal(a, b)
    x0 = _normed(h1, m["norm_h"], bf)
    want = (lm @ _normed(x0, m["final_norm"], bf)).astype(np.float32)
    np.testing.assert_allclose(a, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())
    # the input gain is applied: the logits without it are measurably different
    wrong = (lm @ _normed(bf(h1 / np.sqrt(np.mean(h1 * h1) + EPS)), m["final_norm"], bf)).astype(np.float32)
    assert np.abs(a - wrong).max() > 1e-3 * np.abs(a).max()
