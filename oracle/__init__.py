"""CPU oracle for the weight-quantized linear layer ``out = x @ dequant(W)^T``.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table or
constant with the HIP library; the two meet only at the seeded inputs of
``synth/``.

Everything here is the plain definition, written out slowly:

* ``oracle.formats`` -- bit-level decode of the storage formats the pages name
  (float8_e4m3fn, packed E2M1 nibbles, bfloat16) and correctly rounded
  conversions from fp64.
* ``oracle.ref``     -- the reference results: fp64 dot products of exactly
  decoded weights and exactly widened activations (W8A16, grouped MoE W8A16,
  W4A16 NVFP4), and exact integer arithmetic plus one fp64 epilogue for W8A8.
* ``oracle.compare`` -- the acceptance rules that decide whether a GPU output
  agrees with a reference result.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
something other than itself (library decoders, hand-derived worked examples
under ``tests/golden/``, closed forms, exact rational brute force).  No function
is left "parity unpinned".
"""

from . import formats, ref, compare  # noqa: F401
