"""Adaptive draft length ("Speculative decoding on Apple Silicon" (OptiQ docs), section "About
depth": raise K after a cycle whose drafts were all accepted, lower it after a rejection).
The oracle's rule is pinned by closed forms; the library's host controller (spec_depth_*)
then follows the oracle step for step on random accept histories."""
import numpy as np
import pytest

from oracle import spec as osp
from speculative_decoding_token_amd import binding as B


def test_oracle_depth_closed_forms():
    # clean cycles walk up by `up` to k_max; rejected ones down by `down` to k_min
    d = osp.AdaptiveDepth(2, 1, 7, up=2, down=1)
    seq = []
    for _ in range(5):
        d.update(d.choose(), d.choose())
        seq.append(d.choose())
    assert seq == [4, 6, 7, 7, 7]
    seq = []
    for _ in range(8):
        d.update(0, d.choose())
        seq.append(d.choose())
    assert seq == [6, 5, 4, 3, 2, 1, 1, 1]
    # a partial accept is a rejection; a cycle without drafts changes nothing
    d = osp.AdaptiveDepth(4, 1, 8)
    d.update(3, 4)
    assert d.choose() == 3
    d.update(0, 0)
    assert d.choose() == 3
    # steps of zero pin K
    d = osp.AdaptiveDepth(3, 0, 8, up=0, down=0)
    for acc in (3, 0, 1):
        d.update(acc, 3)
        assert d.choose() == 3
    # k_min = 0 reaches plain decoding, and stays there (no drafts, no outcome to learn from)
    d = osp.AdaptiveDepth(1, 0, 4)
    d.update(0, 1)
    assert d.choose() == 0
    d.update(0, 0)
    assert d.choose() == 0


@pytest.mark.parametrize("seed", range(5))
def test_library_depth_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    k_max = int(rng.integers(1, 17))
    k_min = int(rng.integers(0, k_max + 1))
    k0 = int(rng.integers(k_min, k_max + 1))
    up, down = int(rng.integers(0, 4)), int(rng.integers(0, 4))
    lib, ref = B.Depth(k0, k_min, k_max, up, down), osp.AdaptiveDepth(k0, k_min, k_max, up, down)
    for _ in range(200):
        k = lib.choose()
        assert k == ref.choose()
        # mostly clean or mostly rejected stretches, so both bounds are reached
        acc = k if rng.random() < 0.55 else int(rng.integers(0, k + 1))
        lib.update(acc, k)
        ref.update(acc, k)


def test_library_depth_rejects_bad_input():
    with pytest.raises(B.SpecError):
        B.Depth(5, 1, 4)
    with pytest.raises(B.SpecError):
        B.Depth(2, 3, 4)
    with pytest.raises(B.SpecError):
        B.Depth(2, 1, 17)
    d = B.Depth(2, 1, 4)
    with pytest.raises(B.SpecError):
        d.update(3, 2)
