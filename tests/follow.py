"""Cycle-by-cycle comparison of a GPU speculative generation with the oracle, conditioned on
the GPU's own outputs.

A generation at bf16 precision meets a decision within the float error every few tokens, after
which two correct runs go separate ways.  Instead of stopping there, each GPU cycle is checked
against the oracle run on the same history: the draft model's lists and drafts (the oracle's
draft forwards fed the GPU's previous drafts), the verify's logits and lists, and the accept
decision; then the oracle takes the GPU's accepted tokens and trims its caches as the GPU did.
Lists are compared against the oracle's within the float error of their logits; the discrete
steps that read them (drafting, accepting) are checked exactly on the GPU's own lists, where
only a margin below 1e-6 excuses a difference."""
import numpy as np
import torch

from oracle import model as om
from oracle import philox as oph
from oracle import sampling as osm
from tests.helpers import assert_rows_close, check_list_row, token_lists


def follow_cycles(eng, n_cycles, K, tspec, tW, tkv, dspec, dW, dkv, hist, temperature, seed, rtol):
    """Runs n_cycles GPU cycles of k = K drafts and checks each.  hist: the token history up to
    and including the last accepted token (position tkv.length).  Checks:
    * the draft model's logits (each draft forward's row, read back after the cycle) within rtol
      of the oracle's draft forwards fed the GPU's previous drafts, its lists against the
      oracle's (check_list_row, within the row's measured logit error, as for the verify), and
      each draft token against a draw from the GPU's own list with the same uniform (the argmax
      under greedy sampling);
    * the verify's logits within rtol and its lists (check_list_row);
    * the accept decision: the oracle's rule on the GPU's own lists and uniforms gives the GPU's
      accepted count and tokens exactly, unless |u - p/q| or a sampling step lies within 1e-6.
    Returns counts of the checks."""
    cnt = dict(draft_lists_exact=0, draft_lists_partial=0, drafts=0, verify_lists_exact=0, verify_lists_partial=0,
               accepts=0, accepts_at_tie=0)
    for r in range(n_cycles):
        c = eng.cycle(1, K, r, keep=True)
        L = tkv.length
        gd = [int(t) for t in c.drafts[0]]
        dlg = eng.draft_logits(1, K)[:, 0].cpu().numpy().astype(np.float64)
        # draft model: feed the history it has not consumed, then the GPU's drafts one by one
        lg = None
        while dkv.length <= L:
            pos = dkv.length
            lg, _ = om.forward_one(dspec, dW, dkv, pos, hist[pos])
            dkv.length = pos + 1
        for j in range(K):
            assert_rows_close(dlg[j][None], lg[None], rtol, "draft logits")
            kind = check_list_row(*c.q[j], lg, float(np.abs(dlg[j] - lg).max()), temperature)
            cnt["draft_lists_" + kind] += 1
            gq = token_lists([c.q[j]])[0]
            if temperature <= 0:
                assert gd[j] == gq.argmax(), (r, j)
            else:
                tok, m = osm.sample(gq.ids, gq.probs, oph.uniform(seed, j + 1, r, 0, oph.STREAM_DRAFT))
                assert tok == gd[j] or m < 1e-6, (r, j, tok, gd[j])
            cnt["drafts"] += 1
            if j + 1 < K:
                pos = dkv.length
                lg, _ = om.forward_one(dspec, dW, dkv, pos, gd[j])
                dkv.length = pos + 1
        # verify over the GPU's drafts
        ref = om.forward_tokens(tspec, tW, tkv, [hist[L]] + gd)
        got = c.logits[0].cpu().numpy()
        assert_rows_close(got, ref, rtol)
        abs_err = np.abs(got.astype(np.float64) - ref).max(axis=1)
        for i in range(K + 1):
            cnt["verify_lists_" + check_list_row(*c.p[i], ref[i], abs_err[i], temperature)] += 1
        # accept: the oracle's rule on the GPU's lists
        ps, qs = token_lists(c.p[: K + 1]), token_lists(c.q[:K])
        if temperature <= 0:
            res = osm.accept(gd, qs, ps, True)
        else:
            ua = [oph.uniform(seed, j, r, 0, oph.STREAM_ACCEPT) for j in range(1, K + 1)]
            res = osm.accept(gd, qs, ps, False, ua, oph.uniform(seed, 0, r, 0, oph.STREAM_RESIDUAL))
        if res.margin >= 1e-6:
            assert c.n[0] == res.n and c.tokens[0] == res.tokens, (r, c.n[0], res.n, c.tokens[0], res.tokens)
            cnt["accepts"] += 1
        else:
            cnt["accepts_at_tie"] += 1
        n = c.n[0]
        for kvc in (tkv,):
            kvc.trim(L + 1 + n)
        dkv.trim(min(dkv.length, L + 1 + n))
        hist.extend(int(t) for t in c.tokens[0])
    return cnt
