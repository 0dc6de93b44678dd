"""fp64 CPU oracle for the MAPL boundary codec -- TEST INFRASTRUCTURE ONLY.

This package is the parity reference for the HIP library.  It is plain NumPy
in float64, written from the equations of *Learned Subspace Compression for
Communication-Efficient Pipeline Parallelism* (MAPL), and shares no code,
constants or helpers with the GPU path.  Only the test suite, the graft
entry's smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does.

Every input is widened exactly to float64 (bf16 and fp32 values are exactly
representable), so the oracle applies no intermediate rounding.

Modules
  codec  Eq. (1)-(3) forward maps and their backward (plain definitions).
  spel   Eq. (4)-(7): tangent projection, heavy-ball momentum, Newton-Schulz
         polar for the LMO direction and the retraction (algorithm steps).
  rvq    Section 3.5 residual multi-codebook VQ encode / decode and the
         streaming codebook sync of Appendix F (algorithm steps).

Parity status: every function here is pinned by tests/test_oracle_pins.py
(brute-force loops, closed forms via the SVD, invariants stated on the pages,
library special cases and the paper's printed payload sizes).
"""
from . import codec, spel, rvq  # noqa: F401
