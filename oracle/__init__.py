"""CPU oracle for gated grouped-query causal attention (forward pass).

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check
in ``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything in this package. The HIP library never calls it, and
it never calls the HIP library: the two share no code. The only module both
sides use is the seeded input generator ``gated_gqa_softmax_amd.inputs``,
which contains no attention arithmetic.

Modules:

* ``oracle.attention`` -- the definition written out in NumPy, fp64 by default
  (an fp32 mode exists to reproduce digits a page prints in fp32).
* ``oracle.loops`` -- an independent pure-Python brute force over explicit
  loops, for tiny shapes, used to cross-check ``oracle.attention``.

Parity status of each function is stated in its docstring. The RMSNorm weight
convention and the RoPE pair convention are readings of the pages (the pages
import ``norm.py`` and ``rope.py`` without printing them): those two points
are pinned by invariants and closed forms only, and their agreement with a
real checkpoint's convention is *parity unpinned*.
"""

from . import attention, loops  # noqa: F401
