"""A forward gives the same bits every time: the same draft_step (28-layer 0.6B-shape draft,
first forward over two rows) and the same verify (8B shape cut to 2 layers, K = 4) in fresh
contexts, three times per schedule, compared bit for bit."""
import numpy as np
import pytest
import torch

from speculative_decoding_token_amd import binding as B
from speculative_decoding_token_amd import runtime, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("schedule", ["stream", "step"])
def test_draft_step_is_deterministic(schedule):
    ts = synth.SHAPES["qwen8b"].with_layers(1)
    ds = synth.SHAPES["qwen0p6b"]
    L, k = 2048, 2
    tw = synth.make_weights(ts, 0, device="cuda")
    dw = synth.make_weights(ds, 1, device="cuda")
    tk, tv = synth.make_kv_prefix(ts, L, 0, device="cuda")
    dk, dv = synth.make_kv_prefix(ds, L - 1, 1, device="cuda")
    prev, last = (int(x) for x in synth.make_tokens(2, ds.vocab, 9))
    outs = []
    for rep in range(3):
        eng = runtime.Engine(ts, tw, ds, dw, temperature=0.0, seed=5, max_ctx=L + 40, max_k=k)
        eng.set_schedule(schedule)
        eng.load_prefix(0, 0, tk, tv, L)
        eng.load_prefix(1, 0, dk, dv, L - 1)
        eng.set_last(torch.tensor([last], dtype=torch.int32, device="cuda"),
                     torch.tensor([prev], dtype=torch.int32, device="cuda"))
        buf = eng.buffers(1, k)
        with eng._enter():
            B.draft_step(eng.ctx, 1, k, 0, buf["draft"], buf["q"])
        eng.stream.synchronize()
        lg = eng.draft_logits(1, k)[k - 1, 0].cpu().numpy()
        res = eng.read_buffer(1, B.BUF_RESIDUAL, (1, ds.d_model)).cpu().numpy()[0]
        outs.append((buf["draft"][0].cpu().tolist(), lg, res))
        eng.close()
    for rep in (1, 2):
        same = np.array_equal(outs[rep][1], outs[0][1]) and np.array_equal(outs[rep][2], outs[0][2])
        print(f"draft_step {schedule} run {rep}: drafts {outs[rep][0]} vs {outs[0][0]}, bits "
              f"{'equal' if same else 'DIFFER'} (max logit diff {np.abs(outs[rep][1] - outs[0][1]).max():.3e})")
        assert same and outs[rep][0] == outs[0][0]


@pytest.mark.parametrize("schedule", ["stream", "step", "forward"])
def test_verify_is_deterministic(schedule):
    shape = synth.SHAPES["qwen8b"].with_layers(2)
    L, K = 2048, 4
    w = synth.make_weights(shape, 0, device="cuda")
    k, v = synth.make_kv_prefix(shape, L, 0, device="cuda")
    t0 = int(synth.make_tokens(1, shape.vocab, 7)[0])
    drafts = torch.tensor([[int(x) for x in synth.make_tokens(K, shape.vocab, 8)]], dtype=torch.int32, device="cuda")
    outs = []
    for rep in range(3):
        eng = runtime.Engine(shape, w, temperature=0.0, max_ctx=L + 40, max_k=K)
        eng.set_schedule(schedule)
        eng.load_prefix(0, 0, k, v, L)
        eng.set_last(torch.tensor([t0], dtype=torch.int32, device="cuda"))
        c = eng.cycle(1, K, 0, drafts=drafts, keep=True)
        outs.append(c.logits[0].cpu().numpy())
        eng.close()
    for rep in (1, 2):
        print(f"verify {schedule} run {rep}: max diff {np.abs(outs[rep] - outs[0]).max():.3e}")
        assert np.array_equal(outs[rep], outs[0])
