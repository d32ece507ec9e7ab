"""Benchmark: speculative decoding on one MI355X, 8B-shaped target at K = 4.

Workload: an 8B-shaped bf16 target (36 layers, d 4096, 32 q / 8 kv heads of 128, SwiGLU
12288, vocab 151936) verifying K = 4 drafts from a 0.6B-shaped bf16 draft (28 layers,
d 1024, 16 / 8 heads, SwiGLU 3072, tied head), batch 1, a synthetic 2048-token cache,
random N(0, 0.02) weights.  A step is one cycle of the whole path: draft_step (K draft
forwards), verify_step (one target forward over K+1 rows + truncation), accept, kv_trim,
and the one device-to-host read of the emitted tokens.  The timed host loop keeps the next
cycle queued while it reads the previous cycle's tokens; the same cycles with a wait after
each one are reported beside it.

Prints one JSON line: accepted (emitted) tokens per second over the timed steps (the first of
`--repeats` timed loops; all of them with their median and coefficient of variation under
`repeats`), the verify pass's HBM bytes per second against the 8 TB/s peak and its latency at
every K from 0 to 8, the roofline of the dominant kernel (the gate/up projection + SwiGLU of the
target; the forward kernel when the forward runs as one launch) with its HBM traffic from the
recorded rocprofv3 counters, a teacher-forced upper bound (drafts = the target's own greedy
continuation, every draft accepted), the same cycle sampled (T = 1, top_k 20, top_p 0.95) with
and without the draft-probability control, the adaptive draft length and the cost gate, the
fp8-weight cycle, the linear-attention state step, the stand-alone accept workload (64
sequences, K = 8, the 151936-token vocabulary) against its roofline, the n-gram workload
replayed over a copy-heavy stream after an 8192-token context (the library's lookup and gate,
steps costed with the 9B-shape verify measured at each draft length), the 27B-shape target
with the 0.8B-shape draft (4096-token context, K = 4 cycles, the verify at K = 1, 2, 4, 8, 16)
and the 9B-shape target with its MTP layer drafting (K = 2 cycles, the verify at K = 1..4),
the draft's one- and
two-row projections on the vector ALUs against the MFMA weight-streaming kernels (per-launch
times at M = 1 and 2 and the whole draft_step), and the CPU oracle timed on one full greedy
cycle of the workload after a warm-up cycle.

--weights fp8 runs the same cycle with the target's projections and LM head stored as OCP
E4M3 codes with a float32 scale per output row (one byte per weight instead of two); the
verify's bytes and the dominant kernel's bytes are then counted at that size, and the CPU
baseline is left out.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "accepted tokens/sec + verify-pass HBM GB/s (% peak), 8B-shape K=4, 1 GPU"
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--k", type=int, default=4)
    ap.add_argument("--batch", type=int, default=1,
                    help="sequences speculated together (each its own cache; default 1, the headline config)")
    ap.add_argument("--ctx", type=int, default=2048)
    ap.add_argument("--sampled", action="store_true", help="temperature 1, top_k 20, top_p 0.95")
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-teacher", action="store_true")
    ap.add_argument("--layers", type=int, default=0, help="override target layers (debug only)")
    ap.add_argument("--no-graphs", action="store_true", help="plain launches instead of graph replays")
    ap.add_argument("--schedule", default=None, choices=["step", "stream", "forward"],
                    help="forward schedule of the bf16 models (default: the library's)")
    ap.add_argument("--no-k-sweep", action="store_true", help="skip the verify latency vs K sweep")
    ap.add_argument("--no-ngram", action="store_true", help="skip the n-gram replay on the 9B shape")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 27B (0.8B draft) and 9B (MTP layer) workloads")
    ap.add_argument("--no-crossover", action="store_true",
                    help="skip the draft projections' vector-ALU vs MFMA comparison")
    ap.add_argument("--no-adaptive", action="store_true", help="skip the adaptive draft length runs")
    ap.add_argument("--weights", default="bf16", choices=["bf16", "fp8"],
                    help="target projection weights: bf16, or OCP E4M3 codes with a float32 scale per row")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-weight verify run of the default bench")
    ap.add_argument("--no-sampled", action="store_true", help="skip the sampled-cycle run of the default bench")
    ap.add_argument("--no-accept-workload", action="store_true", help="skip the stand-alone accept workload")
    ap.add_argument("--repeats", type=int, default=5, help="timed loops of --steps cycles (median and CV)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy three times (HBM counter calibration)")
    ap.add_argument("--accept-workload-only", action="store_true",
                    help="only run the stand-alone accept workload (64 sequences, K = 8) and print its figures")
    return ap.parse_args()


def weight_bytes(shape, fp8=False):
    """Streamed weight bytes of one forward: bf16, or one byte per weight plus a float32
    scale per output row."""
    if not fp8:
        return shape.streamed_params() * 2
    rows = shape.n_layers * (shape.q_dim + 2 * shape.kv_dim + 2 * shape.d_model + 2 * shape.d_ffn) + shape.vocab
    return shape.streamed_params() + 4 * rows


def verify_bytes(shape, k, L, batch=1, fp8=False):
    """Algorithmic HBM bytes of one verify: weights once, every sequence's cache read and
    written, logits."""
    M = k + 1
    w = weight_bytes(shape, fp8)
    kv_read = batch * 2 * shape.n_layers * (L + M) * shape.kv_dim * 2
    kv_write = batch * 2 * shape.n_layers * M * shape.kv_dim * 2
    logits = batch * M * shape.vocab * 4
    emb = batch * M * shape.d_model * 2
    return w + kv_read + kv_write + logits + emb


# The dominant kernel of each schedule: the target's gate/up projection + SwiGLU (for the
# one-launch forward, the forward kernel itself), and its HBM bytes per launch from rocprofv3
# FETCH_SIZE / WRITE_SIZE (scaled by a 1 GiB copy's readings) with the sha256 prefix of the
# sources that define it: the figure is reported only while those sources are unchanged.
DOMINANT = {
    "stream": {"kernel": "stream_gemm_kernel<EPI_SWIGLU, 8> (target gate/up + SwiGLU, weights streamed "
                         "through an LDS ring, one workgroup per CU)",
               "slot": "target.gate_up",
               "sources": ["stream_core.h", "stream.hip"], "traffic": 202405029, "sha256": "338e2799e23a26fb"},
    "stream_fp8": {"kernel": "stream_gemm_kernel<EPI_SWIGLU, 4, 1> (target gate/up + SwiGLU over E4M3 weights "
                             "with row scales, streamed through an LDS ring, one workgroup per CU)",
                   "slot": "target.gate_up",
                   "sources": ["stream_core.h", "stream.hip"], "traffic": 101954677, "sha256": "338e2799e23a26fb"},
    "step": {"kernel": "gemm_bf16_kernel<EPI_SWIGLU, 1, NORM, 16> (target gate/up + SwiGLU, one workgroup "
                       "per 16-row tile pair)",
             "slot": "target.gate_up",
             "sources": ["model.hip"], "traffic": None, "sha256": None},
    "forward": {"kernel": "forward_kernel (the whole target forward of the verify as one launch)",
                "slot": "target.forward", "sources": ["forward.hip", "stream_core.h"], "traffic": None,
                "sha256": None},
}
REPS = 8  # back-to-back launches of the dominant kernel between the profiling events (the
          # first REPS - 1 with other layers' weights, so none finds its weights cached)


def sources_sha(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "speculative_decoding_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def dominant_traffic(key):
    d = DOMINANT[key]
    return d["traffic"] if d["sha256"] and sources_sha(d["sources"]) == d["sha256"] else None


def gate_up_bytes(shape, M, fp8=False):
    d, f = shape.d_model, shape.d_ffn
    w = 2 * f * d + 2 * f * 4 if fp8 else 2 * f * d * 2
    return w + M * d * 2 + M * f * 2


def gdn_state_run(torch, synth, B, K, reps=20, layers=48, H=32, dv=128):
    """Linear-attention layer state under speculation (spec_gdn_commit_forward): one launch per
    layer per cycle commits the previous verify's kept tokens (K+1, every draft accepted: the
    most state work) and runs this verify's K+1 tokens.  `layers` states of H heads of
    dv x 128 float32 (2 MB a layer at 32 x 128 x 128), launched back to back on one stream."""
    T = 2 * (K + 1)
    x = synth.make_gdn_inputs(T, H, 128, dv, seed=0, device="cuda")
    states = x["state"].unsqueeze(0).repeat(layers, 1, 1, 1).contiguous()
    out = torch.empty((K + 1, H, dv), device="cuda")
    st = torch.cuda.current_stream()

    def cycle():
        for l in range(layers):
            B.spec_gdn_commit_forward(H, 128, dv, states[l], x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                      K + 1, K + 1, out, st)
    cycle()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        cycle()
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * layers)
    state_bytes = H * dv * 128 * 4
    # state read and written, this call's token rows (q only for the forward half), outputs
    nbytes = 2 * state_bytes + T * H * (128 + dv + 2) * 4 + (K + 1) * H * 128 * 4 + (K + 1) * H * dv * 4
    return {"shape": f"{layers} layers x {H} heads x {dv} x 128 float32 state ({state_bytes / 2**20:.0f} MiB a layer)",
            "tokens_per_launch": f"commit {K + 1} + forward {K + 1}", "us_per_layer": us, "bytes_per_layer": nbytes,
            "GBps": nbytes / (us * 1e-6) / 1e9, "frac_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "timing": f"HIP events around {reps} cycles of {layers} back-to-back launches"}


def cpu_baseline(tshape, dshape, tw, dw, tk, tv, dk, dv, K, prev, last, seed=0):
    """The oracle (numpy, float64 between the contract's rounding points) running the same
    greedy cycle on the host: the draft model's K forwards (its first feeding the tokens at
    positions L-1 and L, as on the GPU), the target's verify over K+1 rows, truncation, accept
    and trim, on the same weights and cache prefixes.  One warm-up cycle, then one timed cycle.
    The weights are widened to float64 once beforehand (host memory, outside the timing)."""
    import numpy as np
    import torch
    from oracle import model as om
    from oracle import sampling as osm
    from oracle import spec as osp

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    t_load = time.perf_counter()

    def host(w):
        conv = lambda t: t.detach().to("cpu").to(torch.float64).numpy()
        out = {"embed": conv(w["embed"]), "final_norm": conv(w["final_norm"]),
               "layers": [{k: conv(v) for k, v in lw.items()} for lw in w["layers"]]}
        out["lm_head"] = out["embed"] if w["lm_head"] is w["embed"] else conv(w["lm_head"])
        return out
    tW, dW = host(tw), host(dw)
    ts, ds = om.Spec.from_shape(tshape), om.Spec.from_shape(dshape)
    L = tk.shape[2]
    tkv = om.KVCache(ts, L + 2 * (K + 1) + 2)
    tkv.load_prefix(tk.double().cpu().numpy(), tv.double().cpu().numpy())
    draft = osp.DraftModel(ds, dW, L + 2 * (K + 1) + 2)
    draft.kv.load_prefix(dk.double().cpu().numpy(), dv.double().cpu().numpy())
    hist = [0] * (L - 1) + [int(prev), int(last)]
    load_s = time.perf_counter() - t_load
    sampler = osp.Sampler(0.0, 20, 0.95)
    times = []
    for rnd in range(2):
        Lr = tkv.length
        t0 = time.perf_counter()
        drafts, qs = draft.propose(hist, Lr, K, sampler, seed, rnd)
        t1 = time.perf_counter()
        ref = om.forward_tokens(ts, tW, tkv, [hist[Lr]] + drafts)
        ps = [osm.truncate(ref[i], 0.0, 20, 0.95) for i in range(K + 1)]
        t2 = time.perf_counter()
        res = osm.accept(drafts, qs, ps, True)
        tkv.trim(Lr + 1 + res.n)
        draft.trim(Lr + 1 + res.n)
        hist.extend(res.tokens)
        t3 = time.perf_counter()
        times.append((t1 - t0, t2 - t1, t3 - t2, len(res.tokens)))
    d_s, v_s, a_s, n_emit = times[-1]
    cycle = d_s + v_s + a_s
    return {
        "value": n_emit / cycle, "unit": "tokens/s", "cores": blas, "kind": "oracle",
        "sample": (f"one full greedy K={K} cycle of the workload after one warm-up cycle: {K} draft forwards of "
                   f"the {dshape.n_layers}-layer draft (the first over 2 rows), the {tshape.n_layers}-layer "
                   f"target's verify over {K + 1} rows with truncation, accept and trim, numpy float64"),
        "cycle_s": cycle, "draft_s": d_s, "verify_s": v_s, "accept_trim_s": a_s, "emitted": n_emit,
        "warmup_cycle_s": sum(times[0][:3]), "weight_widening_s": load_s,
        "os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "blas_threads": blas,
    }


def accept_workload_run(torch, synth, B, batch=64, K=8, sigma=1.0, copies=3, reps=30, seed=0):
    """The accept workload on its own: for `batch` sequences, truncation (T = 1, top_k 20,
    top_p 0.95) of K + 1 target and K draft rows of bf16 logits over the 151936-token vocabulary,
    the drafts sampled from q, and the accept rule with the residual resample; `copies` input
    copies (together larger than the 256 MB memory-side cache) are rotated."""
    V = 151936
    t, d = synth.make_accept_logits(batch, K, V, sigma, seed=seed, device="cuda", copies=copies)
    tl, dl = B.Probs(batch * (K + 1), 20), B.Probs(batch * K, 20)
    nbytes = B.spec_truncate_scratch_size(batch * (K + 1), V)
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    drafts = torch.empty((batch, K), dtype=torch.int32, device="cuda")
    n = torch.empty(batch, dtype=torch.int32, device="cuda")
    out = torch.empty((batch, K + 1), dtype=torch.int32, device="cuda")
    smp = B.sampler(1.0, 20, 0.95)
    st = torch.cuda.current_stream()

    def call(c, rnd, parts=None):
        if parts is not None:
            parts[0].record(st)
        B.spec_truncate(t[c], B.DTYPE_BF16, batch * (K + 1), V, V, smp, tl, None, scratch, nbytes)
        B.spec_truncate(d[c], B.DTYPE_BF16, batch * K, V, V, smp, dl, None, scratch, nbytes)
        if parts is not None:
            parts[1].record(st)
        B.spec_sample(dl, batch, K, seed, rnd, 0, drafts)
        B.spec_accept_lists(drafts, dl, tl, batch, K, False, seed, rnd, n, out, None)
        if parts is not None:
            parts[2].record(st)
    for r in range(copies):
        call(r, r)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for r in range(reps):
        call(r % copies, r)
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    tr, ac = [], []
    for r in range(reps):
        call(r % copies, r, ev)
        torch.cuda.synchronize()
        tr.append(ev[0].elapsed_time(ev[1]) * 1e3)
        ac.append(ev[1].elapsed_time(ev[2]) * 1e3)
    nb = 2 * batch * (2 * K + 1) * V
    acc = float(n.float().mean().item()) / K
    return {"batch": batch, "k": K, "sigma": sigma, "vocab": V, "copies": copies,
            "bytes_per_call": nb, "us_per_call": us, "GBps": nb / (us * 1e-6) / 1e9,
            "frac_peak": nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "roofline_us": nb / (PEAK_HBM_GBS * 1e9) * 1e6,
            "truncate_us": sorted(tr)[len(tr) // 2], "sample_accept_us": sorted(ac)[len(ac) // 2],
            "acceptance_last_call": acc,
            "timing": f"HIP events around {reps} calls back to back (rotating {copies} input copies); the "
                      f"split into truncation and sample + accept is the median of single calls"}


def config_run(torch, synth, runtime, name, tshape, dshape, L, ks, k_cycle, cycles=12, reps=5, drafter=None):
    """One more workload of the pages at its full size: cycles per second at k_cycle (greedy,
    graph replay, HIP events around each call, the first cycles untimed) and the verify's
    latency and HBM rate at each k in ks (explicit drafts, or with the MTP drafter, which
    catches up from every verify, its own drafts; the verify timed alone either way)."""
    t0 = time.perf_counter()
    tw = synth.make_weights(tshape, 0, device="cuda")
    dw = synth.make_weights(dshape, 0, device="cuda") if dshape is not None else None
    tk, tv = synth.make_kv_prefix(tshape, L, 0, device="cuda")
    kmax = max(max(ks), k_cycle)
    max_ctx = L + (cycles + 2 + reps * len(ks)) * (kmax + 1) + 8
    eng = runtime.Engine(tshape, tw, dshape, dw, temperature=0.0, seed=0, max_ctx=max_ctx, max_k=kmax,
                         drafter=drafter)
    eng.load_prefix(0, 0, tk, tv, L)
    st = synth.make_tokens(2, tshape.vocab, 0, tag="start")
    hidden = None
    if dshape is not None:
        dk, dv = synth.make_kv_prefix(dshape, L - 1, 0, device="cuda")
        eng.load_prefix(1, 0, dk, dv, L - 1)
    if drafter == "mtp":
        # the head's own cache over the same prefix, and a hidden row standing in for the
        # target's at L - 1
        mk, mv = synth.make_kv_prefix(tshape, L, 0, device="cuda", tag="mtp-prefix", n_layers=1)
        eng.load_prefix(2, 0, mk, mv, L)
        g = torch.Generator(device="cpu").manual_seed(5)
        hidden = torch.randn((1, tshape.d_model), generator=g, dtype=torch.float32).cuda()
    eng.set_last(torch.tensor([int(st[1])], dtype=torch.int32, device="cuda"),
                 torch.tensor([int(st[0])], dtype=torch.int32, device="cuda"), hidden=hidden)
    ev, rnd = {}, 0
    out = {"target": f"{tshape.name}: {tshape.n_layers} layers, d {tshape.d_model}, {tshape.n_q_heads}/"
                     f"{tshape.n_kv_heads} heads, FFN {tshape.d_ffn}, vocab {tshape.vocab}, bf16",
           "drafter": drafter or (f"{dshape.name}: {dshape.n_layers} layers, d {dshape.d_model}" if dshape else "none"),
           "context": L}
    # cycles at k_cycle
    for _ in range(2):
        eng.cycle(1, k_cycle, rnd)
        rnd += 1
    torch.cuda.synchronize()
    tt = time.perf_counter()
    emitted, acc = 0, 0
    for _ in range(cycles):
        c = eng.cycle(1, k_cycle, rnd)
        rnd += 1
        emitted += len(c.tokens[0])
        acc += c.n[0]
    el = time.perf_counter() - tt
    out["cycle"] = {"k": k_cycle, "tok_s": emitted / el, "ms_per_cycle": el / cycles * 1e3,
                    "acceptance": acc / (k_cycle * cycles)}
    vk = {}
    for k in ks:
        d = None
        if k and drafter != "mtp":
            d = torch.from_numpy(synth.make_tokens(k, tshape.vocab, k, tag="vk").astype("int32")).view(1, k).cuda()
        ms = []
        for i in range(reps):
            eng.cycle(1, k, rnd, drafts=d, events=ev)
            rnd += 1
            if i > 0:
                ms.append(ev["verify"][0].elapsed_time(ev["verify"][1]))
        m = sorted(ms)[len(ms) // 2]
        vb = verify_bytes(tshape, k, L)
        vk[str(k)] = {"verify_ms": m, "GBps": vb / (m * 1e-3) / 1e9, "frac_peak": vb / (m * 1e-3) / 1e9 / PEAK_HBM_GBS}
    out["verify_by_k"] = vk
    out["setup_and_run_s"] = time.perf_counter() - t0
    eng.close()
    return out


def ngram_replay_run(torch, synth, runtime, B, n_ctx=8192, n_gen=8192, k_max=8, n_min=3, max_match=16,
                     reps=6, seed=5):
    """The n-gram workload replayed ("Speculative decoding on Apple Silicon" (OptiQ docs),
    sections "N-gram lookup: any model" and "Methodology": conversations replayed through the
    real drafter and gate, each step costed with verify timings measured per draft length).
    A copy-heavy stream of n_ctx + n_gen tokens (synth.make_copy_stream) plays the target's
    output after an n_ctx-token context: at each step the library's n-gram lookup
    (spec_ngram_match, longest-then-latest match of at least n_min tokens over the history so
    far) proposes up to k drafts, where k comes from the library's acceptance gate
    (spec_gate_*, fed the measured costs) or is k_max with the gate off; drafts are accepted
    while they equal the stream's next tokens, and the step emits those plus one.  A step costs
    the 9B-shape verify at the number of drafts found (HIP events, graph replay, an n_ctx-entry
    cache) plus one lookup; plain decoding costs the verify at k = 0 per token."""
    import dataclasses
    import numpy as np
    shape = dataclasses.replace(synth.SHAPES["qwen9b_mtp"], mtp=False)
    stream = synth.make_copy_stream(n_ctx + n_gen, shape.vocab, seed=seed).astype(np.int32)
    w = synth.make_weights(shape, 0, device="cuda")
    L = n_ctx - 1
    kc, vc = synth.make_kv_prefix(shape, L, 0, device="cuda")
    eng = runtime.Engine(shape, w, temperature=0.0, seed=0, max_ctx=n_ctx + reps * (k_max + 1) * (k_max + 2) + 16,
                         max_k=k_max, drafter="ngram", ngram=(n_min, max_match))
    eng.load_prefix(0, 0, kc, vc, L)
    eng.load_history(0, torch.from_numpy(stream[:L].copy()).cuda())
    eng.set_last(torch.tensor([int(stream[L])], dtype=torch.int32, device="cuda"))
    # verify latency per draft length (explicit drafts: the verify alone)
    ev, verify_ms = {}, []
    rnd = 0
    for k in range(k_max + 1):
        d = torch.from_numpy(stream[L + 1: L + 1 + k].copy()).view(1, k).cuda() if k else None
        ms = []
        for i in range(reps):
            eng.cycle(1, k, rnd, drafts=d, events=ev)
            rnd += 1
            if i > 0:
                ms.append(ev["verify"][0].elapsed_time(ev["verify"][1]))
        verify_ms.append(sorted(ms)[len(ms) // 2])
    eng.close()
    del w, kc, vc
    # the lookup at every position of the generated part, k_max drafts each (a shorter k takes
    # a prefix: the match does not depend on k), contexts as rows of the stream
    N = n_ctx + n_gen
    full = torch.from_numpy(stream.copy()).cuda()
    bt = 256
    ctx = full.view(1, N).expand(bt, N).contiguous()
    drafts_all = np.zeros((n_gen, k_max), np.int32)
    found_all = np.zeros(n_gen, np.int32)
    dr = torch.empty((bt, k_max), dtype=torch.int32, device="cuda")
    nf = torch.empty(bt, dtype=torch.int32, device="cuda")
    mt = torch.empty((bt, 2), dtype=torch.int32, device="cuda")
    for t0 in range(0, n_gen, bt):
        n = min(bt, n_gen - t0)
        lens = torch.arange(n_ctx + t0, n_ctx + t0 + bt, dtype=torch.int32, device="cuda")
        B.spec_ngram_match(ctx, lens, bt, N, k_max, n_min, max_match, dr, nf, mt)
        torch.cuda.synchronize()
        drafts_all[t0:t0 + n] = dr[:n].cpu().numpy()
        found_all[t0:t0 + n] = nf[:n].cpu().numpy()
    # one lookup's time over the whole history (one sequence)
    l1 = torch.tensor([N - 1], dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lk = []
    for _ in range(reps):
        e0.record()
        B.spec_ngram_match(ctx[:1].contiguous(), l1, 1, N, k_max, n_min, max_match, dr, nf, mt)
        e1.record()
        torch.cuda.synchronize()
        lk.append(e0.elapsed_time(e1))
    lookup_ms = sorted(lk)[len(lk) // 2]

    def replay(gate_on):
        # the lookup costs a step, not a draft: the gate's per-draft cost is zero
        gate = B.Gate(k_max, verify_ms, 0.0, gate_on)
        t, cost, steps, drafted, accepted = 0, 0.0, 0, 0, 0
        while t < n_gen:
            k = gate.choose()
            f = int(min(found_all[t], k))
            a = 0
            while a < f and t + a < n_gen and drafts_all[t, a] == stream[n_ctx + t + a]:
                a += 1
            gate.update(a, f)
            cost += verify_ms[f] + (lookup_ms if k > 0 else 0.0)
            drafted += f
            accepted += a
            steps += 1
            t += a + 1
        return {"tok_s": t / cost * 1e3, "steps": steps, "tokens_per_step": t / steps,
                "drafts_per_step": drafted / steps, "acceptance": accepted / drafted if drafted else 0.0}

    plain = 1e3 / verify_ms[0]
    g, ng = replay(True), replay(False)
    return {"target": "9B shape (32 layers, d 4096, 32/8 heads, FFN 12288, vocab 151936), bf16",
            "context": n_ctx, "generated": n_gen, "n_min": n_min, "max_match": max_match, "k_max": k_max,
            "stream": "synth.make_copy_stream: 32-256-token spans, 40% copies of earlier windows, 60% uniform",
            "verify_ms_by_k": verify_ms, "lookup_ms": lookup_ms, "plain_tok_s": plain,
            "gate": dict(g, speedup=g["tok_s"] / plain), "no_gate": dict(ng, speedup=ng["tok_s"] / plain),
            "how": "the stream plays the target's output; drafts accepted while equal to it; each step costs "
                   "the measured verify at the drafts found plus one lookup"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (sharding across "
              f"GPUs is described, not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    from speculative_decoding_token_amd import runtime, synth

    if args.accept_workload_only:
        from speculative_decoding_token_amd import binding as SB
        print(json.dumps({"accept_workload": accept_workload_run(torch, synth, SB)}), flush=True)
        return

    if args.calibrate_copy:
        n = 1 << 30
        x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}), flush=True)
        return

    K = args.k
    tshape = synth.SHAPES["qwen8b"]
    if args.layers:
        tshape = tshape.with_layers(args.layers)
    dshape = synth.SHAPES["qwen0p6b"]
    L = args.ctx
    temp = 1.0 if args.sampled else 0.0
    t_setup = time.perf_counter()
    fp8 = args.weights == "fp8"
    tw = synth.make_weights_fp8(tshape, 0, device="cuda") if fp8 else synth.make_weights(tshape, 0, device="cuda")
    dw = synth.make_weights(dshape, 0, device="cuda")
    tk, tv = synth.make_kv_prefix(tshape, L, 0, device="cuda")
    dk, dv = synth.make_kv_prefix(dshape, L - 1, 0, device="cuda")
    SWEEP_K, SWEEP_REPS = (1, 2, 3, 4, 5, 6, 7, 8, 0), 6  # K = 0 (no draft) last: the draft cache then lags
    CROSS_P, CROSS_T = 3, 6  # draft-projection comparison: profiled cycles per K, timed cycles
    CROSS_CYCLES = 2 * (2 + 2 * CROSS_P + CROSS_T + 1)
    max_k = max(K, max(SWEEP_K))
    n_cycles = args.warmup + (2 + args.repeats) * args.steps + args.profile_steps + 2  # timed runs + sync loop
    max_ctx = L + n_cycles * (K + 1) + len(SWEEP_K) * SWEEP_REPS * (max_k + 1) + CROSS_CYCLES * (K + 1) + 8
    Bn = args.batch
    if Bn > 1:
        if Bn * (K + 1) > 16:
            print("bench.py: batch x (K + 1) rows must stay within 16", file=sys.stderr)
            sys.exit(2)
        max_k = K  # no K sweep for a batch
    eng = runtime.Engine(tshape, tw, dshape, dw, temperature=temp, seed=0, max_ctx=max_ctx, max_k=max_k,
                         max_batch=Bn)
    starts = [synth.make_tokens(2, tshape.vocab, b, tag="start") for b in range(Bn)]

    def reset(e=None):
        e = e or eng
        for b in range(Bn):
            e.load_prefix(0, b, tk, tv, L)
            e.load_prefix(1, b, dk, dv, L - 1)
        e.set_last(torch.tensor([int(st[1]) for st in starts], dtype=torch.int32, device="cuda"),
                   torch.tensor([int(st[0]) for st in starts], dtype=torch.int32, device="cuda"))

    if args.no_graphs:
        eng.use_graphs(False)
    sched = args.schedule or "stream"
    eng.set_schedule(sched)
    reset()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    ev = {}
    rnd = 0
    eng.run(Bn, K, rnd, args.warmup)
    rnd += args.warmup
    torch.cuda.synchronize()
    # no garbage-collector pass inside the timed loops (a pass over the process's objects can
    # stall the host loop for tens of ms); collected before each loop instead
    import gc
    gc.collect()
    gc.disable()
    # timed: the host loop keeps one cycle queued ahead (Engine.run); every cycle's tokens
    # are read back to the host inside the timed region
    t0 = time.perf_counter()
    cycles = eng.run(Bn, K, rnd, args.steps, time_verify=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    rnd += args.steps
    emitted = sum(len(t) for c in cycles for t in c.tokens)
    accepted = sum(sum(c.n) for c in cycles)
    verify_ms = [c.verify_ms for c in cycles]
    # the same cycles with the host waiting for each cycle's tokens before queuing the next
    t1 = time.perf_counter()
    emitted_sync = 0
    for _ in range(args.steps):
        emitted_sync += sum(len(t) for t in eng.cycle(Bn, K, rnd).tokens)
        rnd += 1
    torch.cuda.synchronize()
    sync_loop = {"tok_s": emitted_sync / (time.perf_counter() - t1),
                 "ms_per_step": (time.perf_counter() - t1) / args.steps * 1e3}
    # repeats of the timed loop (the first one is the headline value)
    rep_tok_s = [emitted / elapsed]
    for _ in range(args.repeats - 1):
        torch.cuda.synchronize()
        gc.enable()
        gc.collect()
        gc.disable()
        tr0 = time.perf_counter()
        cyc_r = eng.run(Bn, K, rnd, args.steps)
        torch.cuda.synchronize()
        rep_tok_s.append(sum(len(t) for c in cyc_r for t in c.tokens) / (time.perf_counter() - tr0))
        rnd += args.steps
    gc.enable()
    srt = sorted(rep_tok_s)
    mean = sum(rep_tok_s) / len(rep_tok_s)
    cv = (sum((x - mean) ** 2 for x in rep_tok_s) / len(rep_tok_s)) ** 0.5 / mean
    repeats = {"tok_s": rep_tok_s, "median": srt[len(srt) // 2], "cv": cv,
               "how": f"{len(rep_tok_s)} timed loops of {args.steps} cycles (the first is `value`)"}
    tok_s = emitted / elapsed
    verify_avg_ms = sum(verify_ms) / len(verify_ms)
    vbytes = verify_bytes(tshape, K, L + args.warmup + 1, Bn, fp8)
    verify_gbs = vbytes / (verify_avg_ms * 1e-3) / 1e9

    # verify latency against K (the pass streams the same weights at any K up to 16 rows)
    verify_vs_k = {}
    if not args.no_k_sweep and Bn == 1:
        for k in SWEEP_K:
            ms = []
            for i in range(SWEEP_REPS):
                eng.cycle(1, k, rnd, events=ev)
                rnd += 1
                if i > 0:  # the first cycle at a new K captures its graphs
                    ms.append(ev["verify"][0].elapsed_time(ev["verify"][1]))
            vb = verify_bytes(tshape, k, L, 1, fp8)
            verify_vs_k[str(k)] = {"ms": sum(ms) / len(ms), "GBps": vb / (sum(ms) / len(ms) * 1e-3) / 1e9}

    # per-kernel durations with events around every launch (separate steps); the dominant
    # kernel goes out REPS times back to back between its events (other layers' weights first),
    # so its average carries one dispatch delay per REPS launches
    dom_key = "stream_fp8" if fp8 else sched  # fp8 weights run the streamed projections always
    dom = DOMINANT[dom_key]
    eng.profile(True)
    if dom["slot"] != "target.forward":
        eng.profile_repeat(dom["slot"], REPS)
    for _ in range(args.profile_steps):
        eng.cycle(Bn, K, rnd)
        rnd += 1
    prof = eng.profile_read() if args.profile_steps else {}
    if dom["slot"] != "target.forward":
        eng.profile_repeat(dom["slot"], 1)
    eng.profile(False)
    # The draft's one- and two-row projections on the vector ALUs (the default) against the MFMA
    # weight-streaming kernels the target uses: per-launch times at M = 2 (the first forward of a
    # draft_step, the catch-up row and the new one) and M = 1 (the others), and the whole
    # draft_step at K, HIP events around each launch.
    crossover = None
    if not args.no_crossover and Bn == 1 and sched == "stream" and K >= 2:
        classes = ("qkv", "o_proj", "gate_up", "down", "lm_head")
        crossover = {"how": f"per-launch µs by HIP events over {CROSS_P} profiled cycles at K = 1 (M = 2) "
                            f"and K = {K} (one M = 2 forward, then M = 1), draft_step ms by events over "
                            f"{CROSS_T} graph-replayed cycles"}
        for kind, on in (("vector_alu", True), ("mfma_stream", False)):
            eng.use_gemv(on)
            eng.cycle(1, 1, rnd)
            eng.cycle(1, K, rnd + 1)
            rnd += 2
            eng.profile(True)
            for _ in range(CROSS_P):
                eng.cycle(1, 1, rnd)
                rnd += 1
            p1 = eng.profile_read()
            for _ in range(CROSS_P):
                eng.cycle(1, K, rnd)
                rnd += 1
            pk = eng.profile_read()
            eng.profile(False)
            row = {}
            for c in classes:
                a, b = p1.get("draft." + c), pk.get("draft." + c)
                if not a or not b:
                    continue
                t2 = a["ms"] / a["launches"]
                n1 = b["launches"] - a["launches"]
                t1 = (b["ms"] - a["launches"] * t2) / n1 if n1 > 0 else float("nan")
                row[c] = {"M2_us": t2 * 1e3, "M1_us": t1 * 1e3}
            ev_c, ms = {}, []
            eng.cycle(1, K, rnd, events=ev_c)
            rnd += 1
            for _ in range(CROSS_T):
                eng.cycle(1, K, rnd, events=ev_c)
                rnd += 1
                ms.append(ev_c["draft"][0].elapsed_time(ev_c["draft"][1]))
            row["draft_step_ms"] = sorted(ms)[len(ms) // 2]
            crossover[kind] = row
        eng.use_gemv(True)
    dprof = prof.get(dom["slot"], {"ms": float("nan"), "launches": 1})
    dom_ms = dprof["ms"] / dprof["launches"]
    # the one-launch forward moves the whole verify's bytes (weights, cache, logits)
    dom_bytes = gate_up_bytes(tshape, Bn * (K + 1), fp8) if dom["slot"] == "target.gate_up" else vbytes
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9

    # teacher-forced upper bound: drafts = the target's own greedy continuation
    teacher = None
    if not args.no_teacher and not args.sampled and Bn == 1:
        reset()
        n_tf = args.steps * (K + 1)
        plain, _ = eng.generate(n_tf + K + 1, 0)
        reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks, cyc = eng.generate(n_tf, K, rnd0=rnd, teacher=plain[0])
        torch.cuda.synchronize()
        tf_elapsed = time.perf_counter() - t0
        teacher = {"tok_s": n_tf / tf_elapsed, "cycles": len(cyc),
                   "all_accepted": all(c.n[0] == K for c in cyc[:-1]),
                   "matches_plain": toks[0] == plain[0][:n_tf]}

    # adaptive draft length (host controller spec_depth: +1 after a clean cycle, -1 after a
    # rejection, K in [1, 8]) on the random draft, and with the target's own continuation as
    # drafts (every cycle clean)
    adaptive = None
    if not args.no_adaptive and not args.sampled and Bn == 1:
        from speculative_decoding_token_amd import binding as B
        adaptive = {"rule": "K += 1 after a clean cycle, K -= 1 after a rejection, K in [1, 8], start K",
                    "k_max": max_k}
        n_ad = args.steps * (K + 1)
        reset()
        depth = B.Depth(K, 1, max_k, 1, 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks, cyc = eng.generate(n_ad, K, rnd0=rnd, gate=depth)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        rnd += len(cyc)
        ks = [len(c.drafts[0]) for c in cyc]
        adaptive["draft_model"] = {"tok_s": n_ad / el, "cycles": len(cyc), "k_last": ks[-1],
                                   "k_mean": sum(ks) / len(ks)}
        if teacher is not None:
            reset()
            plain, _ = eng.generate(n_ad + max_k + 1, 0)
            reset()
            depth = B.Depth(K, 1, max_k, 1, 1)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            toks, cyc = eng.generate(n_ad, K, rnd0=rnd, teacher=plain[0], gate=depth)
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            rnd += len(cyc)
            ks = [len(c.drafts[0]) for c in cyc]
            adaptive["teacher_forced"] = {"tok_s": n_ad / el, "cycles": len(cyc), "k_last": ks[-1],
                                          "k_mean": sum(ks) / len(ks), "matches_plain": toks[0] == plain[0][:n_ad]}

    # the cost gate (spec_gate: the K that maximizes the expected tokens per cycle, 1 + a + ... +
    # a^K for the running acceptance a, over the cycle's cost) driven by this box's measured
    # verify latency at every K and the measured draft step cost
    if adaptive is not None and all(str(k) in verify_vs_k for k in range(max_k + 1)):
        from speculative_decoding_token_amd import binding as B
        vc = [verify_vs_k[str(k)]["ms"] for k in range(max_k + 1)]
        draft_ms = max((elapsed / args.steps * 1e3 - verify_avg_ms) / K, 0.0)
        gate = B.Gate(max_k, vc, draft_ms)
        n_ad = args.steps * (K + 1)
        reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks, cyc = eng.generate(n_ad, K, rnd0=rnd, gate=gate)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        rnd += len(cyc)
        ks = [len(c.drafts[0]) for c in cyc]
        adaptive["cost_gate"] = {"verify_ms_by_k": vc, "draft_step_ms": draft_ms, "tok_s": n_ad / el,
                                 "cycles": len(cyc), "k_first": ks[0], "k_last": ks[-1],
                                 "k_mean": sum(ks) / len(ks),
                                 "note": "a cycle at K = 0 leaves the draft model's cache behind (it "
                                         "catches up two rows per draft_step), which costs acceptance "
                                         "only; the tokens are the target's"}

    # the same cycles with the target's weights as E4M3 codes + row scales (fp8 row of the
    # next steps; not the headline): verify latency and rate at the fp8 byte count
    fp8_run = None
    if not fp8 and not args.no_fp8 and Bn == 1:
        tw8 = synth.make_weights_fp8(tshape, 0, device="cuda")
        eng8 = runtime.Engine(tshape, tw8, dshape, dw, temperature=temp, seed=0, max_ctx=max_ctx, max_k=K)
        if args.no_graphs:
            eng8.use_graphs(False)
        reset(eng8)
        eng8.run(1, K, 0, args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        c8 = eng8.run(1, K, args.warmup, args.steps, time_verify=True)
        torch.cuda.synchronize()
        el8 = time.perf_counter() - t0
        n8 = sum(len(t) for c in c8 for t in c.tokens)
        ms8 = [c.verify_ms for c in c8]
        vb8 = verify_bytes(tshape, K, L + args.warmup + 1, 1, True)
        v8 = sum(ms8) / len(ms8)
        fp8_run = {"target_weights": "fp8_e4m3_row", "tok_s": n8 / el8, "verify_ms": v8, "verify_bytes": vb8,
                   "verify_GBps": vb8 / (v8 * 1e-3) / 1e9, "frac_peak": vb8 / (v8 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                   "verify_speedup_vs_bf16": verify_avg_ms / v8}
        del eng8, tw8
        torch.cuda.empty_cache()

    # the same cycle under sampling (T = 1, top_k 20, top_p 0.95): a second context on the same
    # weights
    sampled = None
    if not args.sampled and not fp8 and not args.no_sampled and Bn == 1:
        engs = runtime.Engine(tshape, tw, dshape, dw, temperature=1.0, seed=0, max_ctx=max_ctx, max_k=K)
        if args.no_graphs:
            engs.use_graphs(False)
        engs.set_schedule(sched)
        reset(engs)
        engs.run(1, K, 0, args.warmup)
        torch.cuda.synchronize()
        ts0 = time.perf_counter()
        cs = engs.run(1, K, args.warmup, args.steps, time_verify=True)
        torch.cuda.synchronize()
        els = time.perf_counter() - ts0
        sampled = {"sampler": "T=1 top_k 20 top_p 0.95, Philox uniforms", "tok_s": sum(len(t) for c in cs for t in c.tokens) / els,
                   "ms_per_step": els / args.steps * 1e3, "verify_ms": sum(c.verify_ms for c in cs) / len(cs),
                   "acceptance": sum(c.n[0] for c in cs) / (K * args.steps)}
        # the same sampled cycles with the draft-probability control: the draft stops at its
        # first draft whose list gives it less than p_min, and the device skips the rest of
        # the draft_step's forwards
        if not args.no_adaptive:
            ctl = {}
            for p_min in (0.5,):
                engs.set_draft_controls(p_min, 0)
                reset(engs)
                engs.run(1, K, 0, args.warmup)
                st0 = engs.stats()
                torch.cuda.synchronize()
                ts0 = time.perf_counter()
                cs = engs.run(1, K, args.warmup, args.steps)
                torch.cuda.synchronize()
                els = time.perf_counter() - ts0
                st1 = engs.stats()
                ctl[str(p_min)] = {"tok_s": sum(len(t) for c in cs for t in c.tokens) / els,
                                   "ms_per_step": els / args.steps * 1e3,
                                   "drafts_checked_per_cycle": (st1["drafts_attempted"] - st0["drafts_attempted"]) /
                                                               (st1["cycles"] - st0["cycles"])}
            engs.set_draft_controls(0.0, 0)
            sampled["draft_probability"] = {"k_max": K, "runs": ctl}
        del engs
        torch.cuda.empty_cache()

    # the adaptive draft length's three parts in one place: the depth controller, the cost gate
    # (greedy engine) and the draft-probability control (sampled engine: greedy lists are one-hot)
    if adaptive is not None and sampled is not None and "draft_probability" in sampled:
        adaptive["draft_probability"] = dict(sampled.pop("draft_probability"),
                                             sampler="T=1 top_k 20 top_p 0.95 (the sampled engine)",
                                             without_control_tok_s=sampled["tok_s"])

    from speculative_decoding_token_amd import binding as SB
    gdn_run = gdn_state_run(torch, synth, SB, K)
    accept_run = accept_workload_run(torch, synth, SB) if not args.no_accept_workload else None
    # the headline workload's peak, before the other workloads allocate their models
    peak_gb = torch.cuda.max_memory_allocated() / 1e9
    ngram_run = ngram_replay_run(torch, synth, runtime, SB) if not args.no_ngram and Bn == 1 and not fp8 else None
    configs = None
    if not args.no_configs and Bn == 1 and not fp8:
        configs = {
            "27b_0p8b": config_run(torch, synth, runtime, "27b", synth.SHAPES["qwen27b"], synth.SHAPES["qwen0p8b"],
                                   4096, (1, 2, 4, 8, 16), 4),
            "9b_mtp": config_run(torch, synth, runtime, "9b_mtp", synth.SHAPES["qwen9b_mtp"], None, 2048,
                                 (1, 2, 3, 4), 2, drafter="mtp"),
        }

    out = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"8B-shape {'fp8-weight (E4M3, row scales) ' if fp8 else ''}bf16 target verify "
                               f"K={K} + 0.6B-shape draft, batch {Bn}, "
                               f"KV context {L}, {'sampled T=1 top_k 20 top_p 0.95' if args.sampled else 'greedy'}, "
                               f"random N(0,0.02) weights" + (f", {tshape.n_layers} layers" if args.layers else ""),
                   "global_batch": Bn, "seq_len": L, "k": K, "schedule": "stream" if fp8 else sched,
                   "target_weights": "fp8_e4m3_row" if fp8 else "bf16", "parallelism": "none (1 GPU)"},
        "acceptance": accepted / (K * args.steps * Bn),
        "verify": {"ms": verify_avg_ms, "bytes": vbytes, "GBps": verify_gbs, "frac_peak": verify_gbs / PEAK_HBM_GBS},
        "verify_vs_k": verify_vs_k,
        "host_loop": {"timed": "one cycle queued ahead of the host's read of the previous cycle's tokens",
                      "sync_each_cycle": sync_loop},
        "repeats": repeats,
        "sampled": sampled,
        "roofline": {"bound": "hbm", "kernel": dom["kernel"],
                     "verify_pass": {"GBps": verify_gbs, "frac": verify_gbs / PEAK_HBM_GBS, "ms": verify_avg_ms,
                                     "bytes": vbytes, "note": "the whole verify_step (one graph launch): the "
                                     "metric's figure; achieved/frac below are the dominant kernel's"},
                     "achieved": dom_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dom_gbs / PEAK_HBM_GBS,
                     "traffic": dominant_traffic(dom_key), "bytes_per_launch": dom_bytes, "avg_launch_ms": dom_ms,
                     "timing": (f"HIP events on the context stream around {REPS} back-to-back launches (the first "
                                f"{REPS - 1} with the next layers' weights, then the real one), "
                                if dom["slot"] != "target.forward" else "HIP events around each launch, ")
                               + f"{args.profile_steps} profiled steps after the timed ones"},
        "kernels": {k: {"avg_us": v["ms"] / v["launches"] * 1e3, "launches_per_step": v["launches"] / args.profile_steps}
                    for k, v in prof.items()},
        "draft_projections": crossover,
        "ngram_replay": ngram_run,
        "configs": configs,
        "teacher_forced": teacher,
        "adaptive_depth": adaptive,
        "fp8_weights": fp8_run,
        "linear_attention_state": gdn_run,
        "accept_workload": accept_run,
        "peak_device_memory_GB": peak_gb,
        "setup_s": setup_s,
    }
    if not args.no_cpu_baseline and Bn == 1 and not fp8:
        del eng
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(tshape, dshape, tw, dw, tk, tv, dk, dv, K, starts[0][0], starts[0][1])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
