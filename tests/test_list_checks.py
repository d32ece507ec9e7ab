"""The list comparison used by the GPU parity tests (tests.helpers.check_list_row) must accept
the oracle's own list, excuse only ids that a decision within the stated logit error can
change, and reject everything else."""
import numpy as np
import pytest

from oracle import sampling as osm
from tests.helpers import check_list_row


def row(seed=0, V=5000):
    return np.random.default_rng(seed).normal(0, 1.3, V).astype(np.float32)


@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_own_list_is_exact(temp):
    z = row()
    o = osm.truncate(z, temp, 20, 0.95)
    assert check_list_row(o.ids, o.probs, z, 1e-6, temp) == "exact"


def test_wrong_id_far_from_the_boundary_fails():
    z = row(1)
    o = osm.truncate(z, 1.0, 20, 0.95)
    ids = o.ids.copy()
    top = int(np.argmax(z))
    ids[ids == top] = int(np.argmin(z))   # the most likely token replaced by the least likely
    with pytest.raises(AssertionError):
        check_list_row(np.sort(ids), o.probs, z, 1e-3, 1.0)


def test_boundary_swap_within_the_error_is_partial_and_outside_fails():
    z = row(2)
    order = np.argsort(-z, kind="stable")
    # make the 20th and 21st logits nearly equal, then give the GPU the 21st instead
    z[order[20]] = z[order[19]] - np.float32(1e-3)
    o = osm.truncate(z, 1.0, 20, 1.0)
    ids = np.sort(np.concatenate([o.ids[o.ids != order[19]], [order[20]]]))
    probs = o.probs.copy()
    assert check_list_row(ids, probs, z, 0.01, 1.0, top_p=1.0) == "partial"
    with pytest.raises(AssertionError):
        check_list_row(ids, probs, z, 1e-5, 1.0, top_p=1.0)


def test_probabilities_outside_the_bound_fail():
    z = row(3)
    o = osm.truncate(z, 1.0, 20, 0.95)
    p = o.probs.astype(np.float64).copy()
    p[0] *= 1.5
    with pytest.raises(AssertionError):
        check_list_row(o.ids, p / p.sum(), z, 1e-4, 1.0)


def test_greedy_argmax_within_the_error_is_partial():
    z = row(4)
    order = np.argsort(-z, kind="stable")
    z[order[1]] = z[order[0]] - np.float32(1e-3)
    assert check_list_row([int(order[1])], [1.0], z, 0.01, 0.0) == "partial"
    with pytest.raises(AssertionError):
        check_list_row([int(order[5])], [1.0], z, 1e-4, 0.0)
