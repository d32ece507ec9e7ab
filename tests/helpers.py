"""Shared test helpers: comparisons against the oracle with the near-tie rules.

Tolerances (stated once here, used by every parity test):
* float32 models: logits and probabilities within 1e-4 of the row's largest magnitude;
* bfloat16 models: within 2e-2 of the row's largest magnitude;
* tokens and list ids are bit-exact, except where a decision's float margin is below the
  near-tie threshold: |u - p/q|, a CDF step or the top_p cut below 1e-6 when both sides
  read the same inputs, and for model outputs a logit gap below twice the largest logit
  error observed on that row, or a probability margin below twice the largest
  probability error observed on that row.
"""
import numpy as np

RTOL_F32 = 1e-4
RTOL_BF16 = 2e-2
NEAR_TIE = 1e-6


def row_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return np.abs(got - ref).max(axis=-1) / scale


def assert_rows_close(got, ref, rtol, what="logits"):
    err = row_rel_err(got, ref)
    assert np.all(err <= rtol), f"{what}: worst row error {err.max():.3e} > {rtol}"
    return float(err.max())


def lists_equal(g_ids, g_p, o, prob_rtol):
    """GPU list (ids, probs) vs an oracle TokenList."""
    if len(g_ids) != len(o.ids) or not np.array_equal(np.asarray(g_ids), o.ids):
        return False
    return bool(np.all(np.abs(np.asarray(g_p, np.float64) - o.probs.astype(np.float64)) <= prob_rtol))


def host_arrays(w):
    """A weight dict of torch tensors (any device) as numpy: uint8 fp8 code tensors stay
    uint8, every other tensor becomes float32 values; nested layer dicts are converted too."""
    def conv(v):
        if v is None:
            return None
        if v.dtype.is_floating_point:
            return v.float().cpu().numpy()
        return v.cpu().numpy()
    out = {k: conv(v) for k, v in w.items() if k not in ("layers", "mtp")}
    out["layers"] = [{k: conv(v) for k, v in lw.items()} for lw in w["layers"]]
    return out
