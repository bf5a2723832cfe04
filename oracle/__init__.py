"""CPU oracle for multi-head latent attention over a shared latent cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path; the only common module is ``mla_inputs`` (seeded input generation).

The oracle is deliberately plain: float64 NumPy, per-head keys and values
materialised from the latent, textbook masked softmax attention.  The GPU path
reaches the same numbers through weight absorption instead.

Parity status: every function is pinned by ``tests/test_oracle_*.py``
(brute-force scalar loops, algebraic identities, rotary-embedding invariants,
closed forms of softmax special cases, library cross-checks and planted
mistakes).  The rotary pairing/frequency convention and the INT4 rounding
conventions are readings, not facts printed by the pages: they bind both
paths, and no value printed by the pages pins them (parity unpinned there).
"""
from . import int4, mla  # noqa: F401
