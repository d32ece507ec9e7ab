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


def host_weights_f64(w):
    """A weight dict of torch tensors (any device) as float64 numpy arrays, converted once (the
    oracle's arithmetic is float64; widening here only saves it a conversion per access).  A
    tied LM head stays one array."""
    import torch

    def conv(v):
        return None if v is None else v.detach().to("cpu").to(torch.float64).numpy()
    out = {"embed": conv(w["embed"]), "final_norm": conv(w["final_norm"])}
    out["lm_head"] = out["embed"] if w["lm_head"] is w["embed"] else conv(w["lm_head"])
    out["layers"] = [{k: conv(v) for k, v in lw.items()} for lw in w["layers"]]
    out["mtp"] = None if w.get("mtp") is None else {k: conv(v) for k, v in w["mtp"].items()}
    return out


def bf16_flip_rate(got, ref):
    """Fraction of elements of two arrays of bf16 values that differ."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.mean(got != ref))


def rel_rms(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean((got - ref) ** 2) / max(np.mean(ref ** 2), 1e-300)))


def check_list_row(gpu_ids, gpu_probs, ref_logits, abs_err, temperature, top_k=20, top_p=0.95):
    """Compare one truncated list of the GPU with the oracle's truncation of the oracle's logits
    row, for model outputs that carry a float error; ``abs_err`` bounds |GPU - oracle| on the
    row's logits.  Returns "exact" when every decision of the row lies outside the error and
    the lists were compared whole: the oracle's ids exactly, probabilities within the change
    the logit error can cause (a softmax entry moves by at most 2 p max|dz|).  Returns
    "partial" when a decision lies within the error (the argmax, the top_k boundary or the top_p
    cut): then only the ids whose membership that decision cannot change are compared, i.e. the
    two lists may differ only in ids whose scaled logit lies within twice the error of the
    deciding one (or, at the top_p cut, in the last kept / first dropped id), and the
    probabilities of the shared ids, renormalized over them, must agree within the bound."""
    from oracle import sampling as osm

    z = np.asarray(ref_logits, np.float64)
    o = osm.truncate(np.asarray(ref_logits), temperature, top_k, top_p)
    gi = np.asarray(gpu_ids, np.int64)
    gp = np.asarray(gpu_probs, np.float64)
    T = temperature if temperature > 0 else 1.0
    dz = abs_err / T
    zs = z / T
    pbound = 2.0 * float(np.max(o.probs)) * dz
    tie_k = o.gap_logit < 2 * dz
    tie_p = False
    order = np.argsort(-zs, kind="stable")
    n_keep = len(o.ids)
    cut = []
    if temperature > 0:
        kk = min(top_k, len(zs)) if top_k > 0 else len(zs)
        cut = [zs[order[n_keep - 1]]] + ([zs[order[n_keep]]] if n_keep < kk else [])
        # the cut moves if the running sum is within the error of top_p, or if the last kept and
        # the first dropped token can change places
        tie_p = o.margin < 2 * pbound or (len(cut) == 2 and cut[0] - cut[1] < 2 * dz)
    if not tie_k and not tie_p:
        if not np.array_equal(gi, o.ids):
            d = sorted(set(gi.tolist()) ^ set(o.ids.tolist()))
            raise AssertionError(f"ids differ at {d}: oracle scaled logits {[round(float(z[t]) / T, 5) for t in d]}, "
                                 f"gap {o.gap_logit:.4g}, margin {o.margin:.4g}, error band {dz:.4g}")
        np.testing.assert_allclose(gp, o.probs.astype(np.float64), atol=4.0 * pbound + 1e-6)
        return "exact"
    if temperature <= 0:
        # the GPU's argmax is one of the ids within twice the error of the oracle's maximum
        assert zs[gi[0]] >= zs.max() - 2 * dz, (int(gi[0]), int(o.ids[0]))
        return "partial"
    # ids that a decision within the error may add or drop: those within twice the error of
    # the top_k boundary, and those within twice the error of the top_p cut (plus the last
    # kept and first dropped ids when the running sum itself is within the error)
    kth = zs[order[min(top_k, len(zs)) - 1]]
    amb = set(np.nonzero(np.abs(zs - kth) <= 2 * dz)[0].tolist()) if tie_k else set()
    if tie_p:
        for zc in cut:
            amb.update(np.nonzero(np.abs(zs - zc) <= 2 * dz)[0].tolist())
        amb.update(int(t) for t in order[max(n_keep - 1, 0): n_keep + 1])
    diff = set(gi.tolist()) ^ set(o.ids.tolist())
    assert diff <= amb, (sorted(diff - amb), list(gi), list(o.ids))
    common, ig, io = np.intersect1d(gi, o.ids, return_indices=True)
    assert len(common) >= 1
    a = gp[ig] / gp[ig].sum()
    b = o.probs[io].astype(np.float64) / float(o.probs[io].astype(np.float64).sum())
    np.testing.assert_allclose(a, b, atol=8.0 * pbound + 1e-6)
    return "partial"


def token_lists(lists):
    """GPU (ids, probs) lists as oracle TokenLists (same ids and float32 probabilities)."""
    from oracle import sampling as osm
    return [osm.TokenList(np.asarray(i, np.int64), np.asarray(p, np.float32)) for i, p in lists]
