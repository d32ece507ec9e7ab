"""Full-depth parity of the headline configuration: the 36-layer 8B-shape target verifying
K = 4 drafts over a 2048-entry cache ("Speculative Decoding on Apple Silicon: 119% Faster...",
section "The original result: Qwen3-8B and a 0.6B draft"), greedy and sampled, in the launch
configuration bench.py times (streamed projections, graph replay), and one draft_step of the
28-layer 0.6B-shape draft.  Every RMSNorm gain is drawn from N(1, 0.1).

Two float32 evaluations of the bf16 contract drift apart with depth: a float32 rounding
difference tips a value near a bf16 midpoint to the other neighbour, each projection spreads
one tipped input over all its outputs, and after a few layers most bf16 intermediates of two
correct evaluations differ by an ulp.  So the checks are layered:
* every layer, fed the GPU's own input rows (the residual rows after the layer before, read
  back from a forward of the first l layers), against the oracle's layer on those rows: within
  the bf16 tolerance, per layer;
* the final norm, vocabulary projection and truncation on the GPU's final residual rows
  against the oracle's on the same rows: logits within the tolerance, lists with
  check_list_row;
* end to end against the float64 oracle, bounded by the contract's own drift on these inputs:
  the distance between the oracle evaluated in float32 and in float64 (``Spec.arith32``).
The oracle's weights are widened to float64 once (host memory only, not its arithmetic)."""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import sampling as osm
from speculative_decoding_token_amd import binding as B
from speculative_decoding_token_amd import runtime, synth
from tests.helpers import RTOL_BF16, check_list_row, host_weights_f64, row_rel_err

pytestmark = pytest.mark.gpu

L8, K8 = 2048, 4


def log(msg):
    print(msg, flush=True)


def verify_rows(eng, shape, K, drafts):
    buf = eng.buffers(1, K)
    lg = torch.empty((1, K + 1, shape.vocab), dtype=torch.float32, device="cuda")
    with eng._enter():
        buf["draft"].copy_(torch.tensor([drafts], dtype=torch.int32))
        B.verify_step(eng.ctx, buf["draft"], 1, K, lg, buf["p"])
    eng.stream.synchronize()
    return lg[0].cpu().numpy(), buf["p"].to_lists(K + 1)


def layers_prefix(w, n):
    return {"embed": w["embed"], "lm_head": w["lm_head"], "final_norm": w["final_norm"],
            "layers": w["layers"][:n], "mtp": None}


@pytest.fixture(scope="module")
def verify_8b():
    shape = synth.SHAPES["qwen8b"]
    nl, M = shape.n_layers, K8 + 1
    w = synth.make_weights(shape, 0, device="cuda")
    k, v = synth.make_kv_prefix(shape, L8, 0, device="cuda")
    t0 = int(synth.make_tokens(1, shape.vocab, 7)[0])
    drafts = [int(x) for x in synth.make_tokens(K8, shape.vocab, 8)]
    last = torch.tensor([t0], dtype=torch.int32, device="cuda")
    gpu = {}
    for temp in (0.0, 1.0):
        eng = runtime.Engine(shape, w, temperature=temp, max_ctx=L8 + 40, max_k=K8)
        eng.set_schedule("stream")
        eng.load_prefix(0, 0, k, v, L8)
        eng.set_last(last)
        # verify_step captures its launches into a graph and launches that, as in bench.py
        gpu[temp] = verify_rows(eng, shape, K8, drafts)
        if temp == 0.0:
            resid = [None] * (nl + 1)
            resid[nl] = eng.read_buffer(0, B.BUF_RESIDUAL, (M, shape.d_model)).cpu().numpy()
        assert eng.stats()["sync_timeouts"] == 0
        eng.close()
    # the residual rows after each layer l < 36: a forward of the first l layers (the same
    # weights and kernels; its rows after layer l are those of the 36-layer forward)
    for n in range(1, nl):
        sh = shape.with_layers(n)
        eng = runtime.Engine(sh, layers_prefix(w, n), temperature=0.0, max_ctx=L8 + 40, max_k=K8)
        eng.set_schedule("stream")
        eng.load_prefix(0, 0, k[:n], v[:n], L8)
        eng.set_last(last)
        verify_rows(eng, sh, K8, drafts)
        resid[n] = eng.read_buffer(0, B.BUF_RESIDUAL, (M, shape.d_model)).cpu().numpy()
        eng.close()
    log("GPU forwards done")
    spec, spec32 = om.Spec.from_shape(shape), om.Spec.from_shape(shape, arith32=True)
    W = host_weights_f64(w)
    kh, vh = k.double().cpu().numpy(), v.double().cpu().numpy()
    del w, k, v
    torch.cuda.empty_cache()
    rows = [t0] + drafts
    resid[0] = np.stack([W["embed"][t] for t in rows])
    kv = om.KVCache(spec, L8 + K8 + 2)
    kv.load_prefix(kh, vh)
    ref = om.forward_tokens(spec, W, kv, rows)
    log("oracle float64 forward done")
    kv = om.KVCache(spec, L8 + K8 + 2)
    kv.load_prefix(kh, vh)
    ref32 = om.forward_tokens(spec32, W, kv, rows)
    log("oracle float32 forward done")
    # each layer on the GPU's input rows
    kv = om.KVCache(spec, L8 + K8 + 2)
    kv.load_prefix(kh, vh)
    layer_err = np.zeros((nl, M))
    for l in range(nl):
        out = np.stack([om.decoder_layer(spec, W["layers"][l], resid[l][i].astype(np.float64), L8 + i, kv, l)
                        for i in range(M)])
        layer_err[l] = row_rel_err(resid[l + 1], out)
    log("oracle per-layer pass done")
    # final norm + vocabulary projection on the GPU's final rows
    head = np.stack([(W["lm_head"] @ om.round_bf16(om.rmsnorm(resid[nl][i].astype(np.float64), W["final_norm"],
                                                                spec.rms_eps))).astype(np.float32)
                     for i in range(M)])
    return dict(gpu=gpu, ref=ref, ref32=ref32, layer_err=layer_err, head=head)


def test_8b_full_depth_every_layer(verify_8b):
    le = verify_8b["layer_err"]
    worst = le.max(axis=1)
    log(f"8B 36 layers, each on the GPU's input rows: worst row error per layer "
        f"{np.array2string(worst, precision=1)}; worst {worst.max():.2e} at layer {int(worst.argmax())}")
    assert worst.max() <= RTOL_BF16


@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_8b_full_depth_verify(verify_8b, temp):
    logits, plists = verify_8b["gpu"][temp]
    head, ref, ref32 = verify_8b["head"], verify_8b["ref"], verify_8b["ref32"]
    # the head and truncation on the GPU's final rows
    herr = row_rel_err(logits, head)
    abs_err = np.abs(logits.astype(np.float64) - head).max(axis=1)
    checked = sum(check_list_row(*plists[i], head[i], abs_err[i], temp) == "exact" for i in range(K8 + 1))
    # end to end, against the contract's own drift
    err = row_rel_err(logits, ref)
    floor = row_rel_err(ref32, ref)
    log(f"8B 36 layers K={K8} T={temp}: head on the GPU rows {herr.max():.2e}, {checked} of {K8 + 1} lists "
        f"compared; end to end {np.array2string(err, precision=2)} vs the oracle's float32 drift "
        f"{np.array2string(floor, precision=2)}")
    assert herr.max() <= RTOL_BF16
    assert checked >= (K8 + 1) // 2
    assert err.max() <= max(RTOL_BF16, 2.0 * floor.max())


@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_0p6b_full_depth_draft_step(temp):
    """One draft_step of K = 8 at the 0.6B draft shape (28 layers, tied 151936-token head, a
    2047-entry draft cache): each draft decision against the oracle's draft forward
    conditioned on the GPU's previous drafts.  Each draft's logits row (read back after the
    step) lies within the bf16 tolerance of the oracle's, or twice the contract's own float32
    drift on that row (the float32 and float64 oracle logits of the same forward) where that
    is larger; a decision is compared unless its deciding margin lies within twice the row's
    measured logit error."""
    ts = synth.SHAPES["qwen8b"].with_layers(1)
    ds = synth.SHAPES["qwen0p6b"]
    L, K = 2048, 8
    tw = synth.make_weights(ts, 0, device="cuda")
    dw = synth.make_weights(ds, 1, device="cuda")
    tk, tv = synth.make_kv_prefix(ts, L, 0, device="cuda")
    dk, dv = synth.make_kv_prefix(ds, L - 1, 1, device="cuda")
    prev, last = (int(x) for x in synth.make_tokens(2, ds.vocab, 9))
    eng = runtime.Engine(ts, tw, ds, dw, temperature=temp, seed=5, max_ctx=L + 40, max_k=K)
    eng.set_schedule("stream")
    eng.load_prefix(0, 0, tk, tv, L)
    eng.load_prefix(1, 0, dk, dv, L - 1)
    eng.set_last(torch.tensor([last], dtype=torch.int32, device="cuda"),
                 torch.tensor([prev], dtype=torch.int32, device="cuda"))
    buf = eng.buffers(1, K)
    with eng._enter():
        B.draft_step(eng.ctx, 1, K, 0, buf["draft"], buf["q"])
    eng.stream.synchronize()
    drafts = buf["draft"][0].cpu().tolist()
    qlists = buf["q"].to_lists(K)
    dlg = eng.draft_logits(1, K)[:, 0].cpu().numpy().astype(np.float64)
    spec, spec32 = om.Spec.from_shape(ds), om.Spec.from_shape(ds, arith32=True)
    W = host_weights_f64(dw)
    kh, vh = dk.double().cpu().numpy(), dv.double().cpu().numpy()
    kv, kv32 = om.KVCache(spec, L + K + 2), om.KVCache(spec, L + K + 2)
    kv.load_prefix(kh, vh)
    kv32.load_prefix(kh, vh)
    logits = om.forward_tokens(spec, W, kv, [prev, last])[-1]
    l32 = om.forward_tokens(spec32, W, kv32, [prev, last])[-1]
    checked = 0
    for j in range(K):
        drift = float(row_rel_err(l32, logits))
        assert row_rel_err(dlg[j], logits) <= max(RTOL_BF16, 2.0 * drift), j
        err = float(np.abs(dlg[j] - logits).max())
        o = osm.truncate(logits, temp, 20, 0.95)
        gi, gp = qlists[j]
        if temp == 0.0:
            if o.gap_logit > 2 * err:
                assert drafts[j] == int(o.ids[0]), j
                checked += 1
        else:
            checked += check_list_row(gi, gp, logits, err, temp) == "exact"
        if j + 1 < K:
            logits = om.forward_tokens(spec, W, kv, [drafts[j]])[-1]
            l32 = om.forward_tokens(spec32, W, kv32, [drafts[j]])[-1]
    log(f"0.6B 28 layers draft_step T={temp}: {checked} of {K} draft decisions compared whole")
    assert checked >= 1 or temp > 0


@pytest.mark.parametrize("k", [1, 3])
def test_0p6b_full_depth_draft_forward_logits(k):
    """The k-th draft forward of a greedy draft_step (the first runs two rows, the tokens at L-1
    and L; the later ones one row, the previous draft) of the 28-layer 0.6B-shape draft: its
    logits row in the streamed schedule (the vector-ALU projections of one and two rows), in the
    streamed schedule with those projections on the MFMA weight-streaming kernels
    (spec_use_gemv off) and in the per-tile schedule (the MFMA projections), against each other
    and against the oracle fed the same drafts, beside the oracle's own float32 drift."""
    ts = synth.SHAPES["qwen8b"].with_layers(1)
    ds = synth.SHAPES["qwen0p6b"]
    L = 2048
    tw = synth.make_weights(ts, 0, device="cuda")
    dw = synth.make_weights(ds, 1, device="cuda")
    tk, tv = synth.make_kv_prefix(ts, L, 0, device="cuda")
    dk, dv = synth.make_kv_prefix(ds, L - 1, 1, device="cuda")
    prev, last = (int(x) for x in synth.make_tokens(2, ds.vocab, 9))
    got, drafts = {}, {}
    for sched in ("stream", "step", "stream_mfma"):
        eng = runtime.Engine(ts, tw, ds, dw, temperature=0.0, seed=5, max_ctx=L + 40, max_k=k)
        eng.set_schedule("stream" if sched == "stream_mfma" else sched)
        eng.use_gemv(sched != "stream_mfma")
        eng.load_prefix(0, 0, tk, tv, L)
        eng.load_prefix(1, 0, dk, dv, L - 1)
        eng.set_last(torch.tensor([last], dtype=torch.int32, device="cuda"),
                     torch.tensor([prev], dtype=torch.int32, device="cuda"))
        buf = eng.buffers(1, k)
        with eng._enter():
            B.draft_step(eng.ctx, 1, k, 0, buf["draft"], buf["q"])
        eng.stream.synchronize()
        got[sched] = eng.draft_logits(1, k)[k - 1, 0].cpu().numpy()
        drafts[sched] = buf["draft"][0].cpu().tolist()
        eng.close()
    spec, spec32 = om.Spec.from_shape(ds), om.Spec.from_shape(ds, arith32=True)
    W = host_weights_f64(dw)
    kh, vh = dk.double().cpu().numpy(), dv.double().cpu().numpy()
    kv, kv32 = om.KVCache(spec, L + k + 4), om.KVCache(spec, L + k + 4)
    kv.load_prefix(kh, vh)
    kv32.load_prefix(kh, vh)
    # the oracle fed the streamed schedule's drafts
    toks = [prev, last] + drafts["stream"][: k - 1]
    ref = om.forward_tokens(spec, W, kv, toks)[-1]
    r32 = om.forward_tokens(spec32, W, kv32, toks)[-1]
    e_stream = float(row_rel_err(got["stream"], ref))
    e_step = float(row_rel_err(got["step"], ref))
    e_mfma = float(row_rel_err(got["stream_mfma"], ref))
    drift = float(row_rel_err(r32, ref))
    log(f"0.6B 28 layers, draft forward {k}: stream {e_stream:.2e}, step {e_step:.2e}, stream on MFMA "
        f"{e_mfma:.2e} (drafts {'equal' if drafts['stream'] == drafts['step'] == drafts['stream_mfma'] else 'differ'}); "
        f"oracle float32 drift {drift:.2e}")
    assert e_stream <= max(RTOL_BF16, 2.0 * drift)
    for other, e in (("step", e_step), ("stream_mfma", e_mfma)):
        if drafts["stream"] == drafts[other]:
            assert e <= max(RTOL_BF16, 2.0 * drift), other
