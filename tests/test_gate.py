"""The n-gram acceptance gate of the library (host code behind spec_gate_*) against the
oracle's Gate: same draft length after every step and the same acceptance estimate, bit for
bit, on random cost tables and acceptance histories.  The gate's reading of "Speculative
decoding on Apple Silicon" (OptiQ docs), section "N-gram lookup: any model", is pinned on the
oracle side by closed-form cases."""
import numpy as np
import pytest

from oracle import ngram as ong
from speculative_decoding_token_amd import binding as B


@pytest.mark.parametrize("seed", range(6))
def test_gate_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    n_max = int(rng.integers(1, 9))
    base = float(rng.uniform(1.0, 20.0))
    cost = [base * (1.0 + float(x)) for x in np.concatenate([[0.0], np.sort(rng.uniform(0, 0.6, n_max))])]
    draft = float(rng.uniform(0.0, 0.2)) * base
    enabled = bool(seed % 5)
    g_lib = B.Gate(n_max, cost, draft, enabled)
    g_ref = ong.Gate(n_max, cost, draft, enabled)
    for _ in range(60):
        k = g_lib.choose()
        assert k == g_ref.choose()
        assert g_lib.alpha == g_ref.alpha
        att = k if k > 0 else 0
        acc = int(rng.integers(0, att + 1)) if att else 0
        g_lib.update(acc, att)
        g_ref.update(acc, att)


def test_gate_edges():
    g = B.Gate(4, [1.0, 1.1, 1.2, 1.3, 1.4])
    assert g.choose() == 4
    for _ in range(20):
        g.update(0, 4)
    assert g.choose() == 0
    g.update(0, 0)          # a step without drafts leaves alpha alone
    a = g.alpha
    g.update(0, 0)
    assert g.alpha == a
    with pytest.raises(B.SpecError):
        B.Gate(4, [0.0, 1.0, 1.0, 1.0, 1.0])
    with pytest.raises(B.SpecError):
        B.Gate(17, [1.0] * 18)
    with pytest.raises(B.SpecError):
        g.update(3, 2)
