"""Where the GPU-vs-oracle differences of a bf16 verify come from.

The kernels round at exactly the precision contract's points (the normed rows RMSNorm(x) * g,
q, k, v, the attention output, the SwiGLU product to bf16; residual, softmax and logits
float32), so they differ from the float64 oracle only by float32 arithmetic: summation order
in the projections and attention, float32 exp and rsqrt.  Each such difference can tip a
value that lies near the midpoint of two bf16 neighbours to the other one, and every
projection spreads one tipped input over all of its outputs, so the share of tipped elements
grows stage by stage.  This test reads the last layer's intermediates back from the GPU
(spec_debug_read) for a verify at the 8B shape (K = 4 over a 2048-entry cache) cut to one and
to two layers, compares each with the oracle's, and prints per stage the relative rms
difference and, for bf16 quantities, the share of elements that differ.  The first layer's
raw q and k (before any bf16 rounding of the layer) must agree to float32 accuracy; the bars
on the later stages bound the growth the contract itself allows."""
import numpy as np
import pytest
import torch

from oracle import model as om
from speculative_decoding_token_amd import binding as B
from speculative_decoding_token_amd import runtime, synth
from tests.helpers import bf16_flip_rate, host_weights_f64, rel_rms, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_layers", [1, 2])
def test_stage_errors_8b_shape(n_layers):
    shape = synth.SHAPES["qwen8b"].with_layers(n_layers)
    L, K = 2048, 4
    M = K + 1
    w = synth.make_weights(shape, 0, device="cuda")
    k, v = synth.make_kv_prefix(shape, L, 0, device="cuda")
    eng = runtime.Engine(shape, w, temperature=0.0, max_ctx=L + 40, max_k=K)
    eng.set_schedule("stream")
    eng.load_prefix(0, 0, k, v, L)
    t0 = int(synth.make_tokens(1, shape.vocab, 7)[0])
    drafts = [int(x) for x in synth.make_tokens(K, shape.vocab, 8)]
    eng.set_last(torch.tensor([t0], dtype=torch.int32, device="cuda"))
    c = eng.cycle(1, K, 0, drafts=torch.tensor([drafts], dtype=torch.int32, device="cuda"), keep=True)
    logits = c.logits[0].cpu().numpy()
    d, qd, kvd, f = shape.d_model, shape.q_dim, shape.kv_dim, shape.d_ffn
    g = {
        "q_raw": eng.read_buffer(0, B.BUF_Q, (M, qd)).cpu().numpy(),
        "k_raw": eng.read_buffer(0, B.BUF_K, (M, kvd)).cpu().numpy(),
        "o": eng.read_buffer(0, B.BUF_ATTN, (M, qd), torch.bfloat16).float().cpu().numpy(),
        "h": eng.read_buffer(0, B.BUF_SWIGLU, (M, f), torch.bfloat16).float().cpu().numpy(),
        "x_out": eng.read_buffer(0, B.BUF_RESIDUAL, (M, d)).cpu().numpy(),
    }
    cap = (L + 40) + K + 2  # the engine's max_ctx + max_k + 2
    cv = eng.read_buffer(0, B.BUF_CACHE_V, (n_layers, shape.n_kv_heads, cap, shape.head_dim), torch.bfloat16)
    g["v"] = cv[-1, :, L:L + M, :].float().permute(1, 0, 2).reshape(M, kvd).cpu().numpy()
    ck = eng.read_buffer(0, B.BUF_CACHE_K, (n_layers, shape.n_kv_heads, cap, shape.head_dim), torch.bfloat16)
    g["k"] = ck[-1, :, L:L + M, :].float().permute(1, 0, 2).reshape(M, kvd).cpu().numpy()

    spec = om.Spec.from_shape(shape)
    W = host_weights_f64(w)
    kvc = om.KVCache(spec, L + K + 2)
    kvc.load_prefix(k.double().cpu().numpy(), v.double().cpu().numpy())
    traces = []
    ref = om.forward_tokens(spec, W, kvc, [t0] + drafts, traces)
    last = [tr[-1] for tr in traces]
    o = {name: np.stack([t[name] for t in last]) for name in ("q_raw", "k_raw", "k", "v", "o", "h", "x_out")}
    report = {}
    for name in ("q_raw", "k_raw", "k", "v", "o", "h", "x_out"):
        e = rel_rms(g[name], o[name])
        fl = bf16_flip_rate(g[name], o[name]) if name in ("k", "v", "o", "h") else float("nan")
        report[name] = (e, fl)
        print(f"L{n_layers} layer {n_layers - 1} {name:6s} rel rms {e:.2e}  bf16 differing {fl:.3f}")
    lerr = float(row_rel_err(logits, ref).max())
    print(f"L{n_layers} logits worst row error {lerr:.2e}")
    if n_layers == 1:
        # before any bf16 rounding inside the layer only the float32 sums differ (and, rarely, an
        # element of the embedding's normed row tipped by the float32 rsqrt)
        assert report["q_raw"][0] < 1e-4 and report["k_raw"][0] < 1e-4
    assert report["x_out"][0] < 2e-2
    assert lerr < 2e-2
