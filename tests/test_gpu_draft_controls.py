"""GPU parity of the draft controls ("What is Speculative Decoding and How Does a Draft Model
Work?", section "The demo, draft model on and off with two pairings": most drafts, fewest drafts
worth checking, draft probability) against the oracle.

* The tiny float32 pair, generated with the controls on: token streams and the drafts checked
  equal the oracle's run with the same controls.
* The 0.6B-shaped bf16 draft model (2 layers) on each schedule: with a draft probability that
  stops the draft run part-way, the device skips the remaining draft forwards; the cycle's
  tokens must equal the oracle's accept rule applied to the first kept drafts of an unstopped run
  (same draws, same lists), and the drafts counted as attempted to the kept count read off those
  lists with the oracle's rule.
"""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import philox as oph
from oracle import sampling as osm
from oracle import spec as osp
from speculative_decoding_token_amd import runtime, synth
from tests.helpers import token_lists
from tests.test_gpu_model import DS, TS, cmp_streams, prompt_tensor

pytestmark = pytest.mark.gpu
SEED = 1234


def tiny_pair():
    tw = synth.make_weights(TS, 0)
    dw = synth.make_weights(DS, 1, std=1.0)  # peaked draft lists: confidences spread over (0, 1]
    return tw, dw


@pytest.mark.parametrize("temperature,p_min,min_draft", [(1.0, 0.3, 0), (1.0, 0.6, 2), (1.0, 1.0, 0),
                                                         (0.0, 0.0, 5), (0.0, 0.5, 2)])
def test_tiny_generation_with_draft_controls(temperature, p_min, min_draft):
    K, N = 4, 48
    tw, dw = tiny_pair()
    eng = runtime.Engine(TS, synth.weights_to(tw, "cuda"), DS, synth.weights_to(dw, "cuda"),
                         temperature=temperature, seed=SEED, max_ctx=160, max_k=8)
    eng.set_draft_controls(p_min, min_draft)
    p, pt = prompt_tensor()
    eng.prefill(pt)
    toks, cycles = eng.generate(N, K)
    tspec, dspec = om.Spec.from_shape(TS), om.Spec.from_shape(DS)
    tW, dW = synth.weights_to_numpy(tw), synth.weights_to_numpy(dw)
    tkv = om.KVCache(tspec, 160)
    osp.prefill(tspec, tW, tkv, [int(x) for x in p[:-1]])
    d = osp.DraftModel(dspec, dW, 160)
    osp.prefill(dspec, dW, d.kv, [int(x) for x in p[:-1]])
    ref = osp.run(tspec, tW, tkv, int(p[-1]), [int(x) for x in p], N, K, osp.Sampler(temperature, 20, 0.95),
                  SEED, draft=d, p_min=p_min, min_draft=min_draft)
    agree = cmp_streams(toks[0], ref, temperature == 0.0, 2e-4 * 2, 1e-4)
    st = eng.stats()
    kept = [len(c.drafts) for c in ref.cycles]
    print(f"controls T={temperature} p_min={p_min} min_draft={min_draft}: {agree} of {N} tokens agree, "
          f"drafts checked per cycle {kept[:12]}, GPU total {st['drafts_attempted']}")
    assert agree >= N // 2, agree
    if agree == N:
        # the whole run agrees: the same cycles, drafts checked and accepted
        assert len(cycles) == len(ref.cycles)
        assert st["drafts_attempted"] == ref.drafts_attempted
        assert st["drafts_accepted"] == ref.drafts_accepted
    if min_draft > K:
        assert ref.drafts_attempted == 0  # every cycle a plain decoding step


def confidence(ids, probs, tok):
    hit = np.nonzero(np.asarray(ids) == tok)[0]
    return np.float32(probs[hit[0]]) if len(hit) else np.float32(0.0)


@pytest.mark.parametrize("schedule", ["stream", "forward", "step"])
def test_draft_probability_skips_forwards_and_checks_the_kept_drafts(schedule):
    shape = synth.SHAPES["qwen0p6b"].with_layers(2)
    L, K, rnd = 1024, 8, 0
    tw = synth.make_weights(shape, 0, device="cuda")
    dw = synth.make_weights(shape, 1, std=0.08, device="cuda")
    tk, tv = synth.make_kv_prefix(shape, L, 0, device="cuda")
    dk, dv = synth.make_kv_prefix(shape, L - 1, 1, device="cuda")
    prev, last = (int(x) for x in synth.make_tokens(2, shape.vocab, 9))

    def engine():
        e = runtime.Engine(shape, tw, shape, dw, temperature=1.0, seed=SEED, max_ctx=L + 40, max_k=K)
        e.set_schedule(schedule)
        e.load_prefix(0, 0, tk, tv, L)
        e.load_prefix(1, 0, dk, dv, L - 1)
        e.set_last(torch.tensor([last], dtype=torch.int32, device="cuda"),
                   torch.tensor([prev], dtype=torch.int32, device="cuda"))
        return e

    # the unstopped cycle: its drafts, their lists and the target's lists
    a = engine()
    ca = a.cycle(1, K, rnd, keep=True)
    drafts, q, p = ca.drafts[0], ca.q, ca.p
    conf = [confidence(*q[j], drafts[j]) for j in range(K)]
    print(f"{schedule}: draft confidences {[round(float(c), 3) for c in conf]}")
    # thresholds: one that stops part-way (between the smallest and largest of the first drafts'
    # confidences) and one above every confidence (only the first draft forward runs)
    mid = float(np.sort(conf[: K // 2])[len(conf[: K // 2]) // 2])
    for p_min in (mid, 1.0):
        kb = next((j for j in range(K) if not osp.keeps_drafting(token_lists([q[j]])[0], drafts[j], p_min)), K)
        b = engine()
        b.set_draft_controls(p_min, 0)
        cb = b.cycle(1, K, rnd, keep=True)
        st = b.stats()
        assert st["drafts_attempted"] == kb, (p_min, kb, st)
        assert cb.drafts[0][:kb] == drafts[:kb]
        # the accept rule on the kept drafts with the same lists and uniforms
        u_acc = [oph.uniform(SEED, j, rnd, 0, oph.STREAM_ACCEPT) for j in range(1, kb + 1)]
        u_res = oph.uniform(SEED, 0, rnd, 0, oph.STREAM_RESIDUAL)
        res = osm.accept(drafts[:kb], token_lists(q[:kb]), token_lists(p[: kb + 1]), False, u_acc, u_res)
        assert cb.n[0] == res.n and cb.tokens[0] == [int(t) for t in res.tokens], (p_min, kb)
        print(f"{schedule}: p_min {p_min:.3f} kept {kb} of {K} drafts, accepted {res.n}")
