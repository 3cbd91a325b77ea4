"""CPU oracle for the fused MoE expert FFN forward (test infrastructure only).

This package is test infrastructure.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import or
run it; the HIP library never calls into it and shares no code with it.

Everything is plain NumPy in float64 (or exact integer arithmetic) and follows
the pages' description step by step:

* ``formats``  -- OCP FP8 E4M3FN / FP4 E2M1 / E8M0 decoding, BF16 and E4M3
  round-to-nearest-even, and the amax -> UE8M0 requant scale rule.
* ``routing``  -- token -> expert tables (counts, block-padded offsets, slot
  table, inverse table, per-block slack, pull order), twice: naive loops and
  a vectorised stable-argsort twin.
* ``forward``  -- grouped Linear1, SwiGLU x top-k weight, FP8 requant,
  grouped Linear2, FP32 top-k combine written as BF16.

Parity pins: every function is pinned by tests under ``tests/`` marked
``not gpu`` (exhaustive codec tables, library casts, brute force, exact
rational arithmetic, closed-form invariants).  The SiLU step has no printed
value on the pages; it is pinned by an independent per-token reference built
from library routines (torch's float8/bfloat16 casts and
``torch.nn.functional.silu`` in float64), which the whole forward matches bit
for bit.  No function is left unpinned.
"""
from . import formats, routing, forward  # noqa: F401
