"""bench.py's command line on the host: it measures one GPU and says so for any other count
(the check comes before any GPU work), and its byte counts follow the shapes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from speculative_decoding_token_amd import synth  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_verify_bytes_of_the_8b_shape():
    s = synth.SHAPES["qwen8b"]
    # 7.568 G streamed parameters in bf16, the cache read and written, logits and input rows
    b = bench.verify_bytes(s, 4, 2048)
    assert abs(s.streamed_params() * 2 / 1e9 - 15.136) < 1e-3
    assert 15.43e9 < b < 15.45e9
    # fp8: one byte per weight plus a float32 scale per output row
    b8 = bench.verify_bytes(s, 4, 2048, fp8=True)
    assert b - b8 == s.streamed_params() - 4 * (s.n_layers * (s.q_dim + 2 * s.kv_dim + 2 * s.d_model + 2 * s.d_ffn)
                                                + s.vocab)


def test_gate_up_bytes():
    s = synth.SHAPES["qwen8b"]
    assert bench.gate_up_bytes(s, 5) == 201490432
    assert bench.gate_up_bytes(s, 5, fp8=True) == 100925440
