"""Pins of the oracle's linear-attention (gated delta rule) state and its snapshot-and-replay
rollback: an element-by-element loop of the update, the closed form without writes (beta = 0),
the delta rule's exact key-value association for orthonormal keys, causality of the outputs,
and rollback = a run over the kept prefix."""
import numpy as np
import pytest

from oracle import gdn


def rand_inputs(T, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(T, H, dk))
    k = rng.normal(size=(T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(T, H, dv))
    a = rng.uniform(0.8, 1.0, size=(T, H))
    b = rng.uniform(0.1, 0.9, size=(T, H))
    S0 = rng.normal(size=(H, dv, dk)) * 0.3
    return S0, q, k, v, a, b


def test_step_matches_elementwise_loop():
    rng = np.random.default_rng(0)
    dv, dk = 3, 4
    S = rng.normal(size=(dv, dk))
    k = rng.normal(size=dk)
    v = rng.normal(size=dv)
    a, b = 0.9, 0.4
    want = np.zeros((dv, dk))
    for i in range(dv):
        for j in range(dk):
            acc = 0.0
            for l in range(dk):
                acc += S[i, l] * ((1.0 if l == j else 0.0) - b * k[l] * k[j])
            want[i, j] = a * acc + b * v[i] * k[j]
    np.testing.assert_allclose(gdn.step(S, k, v, a, b), want, rtol=0, atol=1e-14)


def test_no_writes_is_pure_decay():
    S0, q, k, v, a, _ = rand_inputs(6, 2, 8, 5, 1)
    b = np.zeros_like(a)
    out, states = gdn.run(S0, q, k, v, a, b)
    decay = np.cumprod(a, axis=0)  # [T, H]
    for t in range(6):
        for h in range(2):
            np.testing.assert_allclose(states[t][h], decay[t, h] * S0[h], rtol=1e-12)
            np.testing.assert_allclose(out[t, h], decay[t, h] * S0[h] @ q[t, h], rtol=1e-12)


def test_orthonormal_keys_are_stored_exactly():
    # alpha = beta = 1: writing v at a unit key overwrites what the state returned for that key;
    # keys orthogonal to it are untouched, so every (key, value) pair is retrievable
    dk, dv, T = 6, 4, 5
    rng = np.random.default_rng(2)
    basis, _ = np.linalg.qr(rng.normal(size=(dk, dk)))
    k = basis[:T][:, None, :]
    v = rng.normal(size=(T, 1, dv))
    q = k.copy()
    S0 = rng.normal(size=(1, dv, dk))
    out, states = gdn.run(S0, q, k, v, np.ones((T, 1)), np.ones((T, 1)))
    S = states[-1][0]
    for t in range(T):
        np.testing.assert_allclose(S @ k[t, 0], v[t, 0], atol=1e-12)
        np.testing.assert_allclose(out[t, 0], v[t, 0], atol=1e-12)  # o_t = S_t k_t = v_t
    # a key orthogonal to all written ones still reads the initial state
    np.testing.assert_allclose(S @ basis[T], S0[0] @ basis[T], atol=1e-12)


def test_outputs_are_causal():
    S0, q, k, v, a, b = rand_inputs(7, 3, 8, 6, 3)
    out, _ = gdn.run(S0, q, k, v, a, b)
    k2, v2 = k.copy(), v.copy()
    k2[4:] = -k2[4:]
    v2[4:] += 1.0
    out2, _ = gdn.run(S0, q, k2, v2, a, b)
    np.testing.assert_array_equal(out[:4], out2[:4])
    assert not np.allclose(out[4:], out2[4:])


@pytest.mark.parametrize("n_keep", [0, 1, 3, 5])
def test_rollback_equals_a_run_over_the_kept_prefix(n_keep):
    S0, q, k, v, a, b = rand_inputs(5, 2, 8, 4, 4)
    out, S = gdn.speculate(S0, q, k, v, a, b, n_keep)
    full_out, states = gdn.run(S0, q, k, v, a, b)
    np.testing.assert_array_equal(out, full_out)  # the speculative outputs do not depend on n_keep
    want = S0 if n_keep == 0 else states[n_keep - 1]
    np.testing.assert_array_equal(S, want)
    _, prefix_states = gdn.run(S0, q[:n_keep], k[:n_keep], v[:n_keep], a[:n_keep], b[:n_keep])
    if n_keep:
        np.testing.assert_array_equal(S, prefix_states[-1])
    with pytest.raises(ValueError):
        gdn.speculate(S0, q, k, v, a, b, 6)
