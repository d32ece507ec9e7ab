"""CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package.  The HIP
library never links, imports or calls it, and it shares no code, constant table or
helper with the HIP path: the two are independent readings of the same pages.

The oracle is plain, slow and written to be checked by eye against the pages:

* ``model``    — the target/draft decoder forward, one token at a time (a verify over
  K+1 positions is K+1 successive single-token forwards), fp64 arithmetic with
  bfloat16 rounding at the points of the precision contract when the model is bf16.
* ``sampling`` — temperature / top-k / top-p truncation, sampling from a list, and the
  accept rule (greedy match, or accept with probability min(1, p/q) and resample from
  the clipped, renormalized difference max(0, p - q)).  All in float32 to take the same
  decisions in the same precision as the kernels.
* ``philox``   — Philox4x32-10, the counter-based generator that supplies every uniform.
* ``ngram``    — n-gram lookup drafting and the acceptance-rate gate.
* ``spec``     — the draft / verify / accept / trim loop and plain greedy decoding.

Parity pins: every function is checked in ``tests/test_oracle_*.py`` against values
the pages print, closed forms, brute force on tiny inputs, or library routines.  The
MTP head architecture is a reading (the pages give no formula): its numerics are
"parity unpinned" beyond the shared decoder invariants.
"""
from . import philox, numerics, sampling, model, ngram, spec  # noqa: F401
