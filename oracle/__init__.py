"""CPU oracle for the selective-scan (S6) hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it and
shares no code with it.

Everything is plain NumPy in float64, serial over time, vectorised over the
independent (batch, channel, state) columns.  Each function names the passage
of the pages it follows.  Pages are cited by title and section:

* "Mamba: Linear-Time Sequence Modeling with Selective State Spaces" -- the
  Arabic reading guide to arXiv 2312.00752 (sections Method, Selection
  mechanism (S6), Hardware-aware state expansion, FAQ).
* "Mamba / MambaMini" -- the Chinese derivation of the parallel scan
  (Step 1 .. Step 4) and its Q&A.
* "Mamba" -- the CSDN tutorial (section 3, state space; section (2) Mamba).

Pinned by the tests under ``tests/test_oracle_*.py`` against closed forms,
brute force, library routines and exact special cases.  Parity unpinned:
nothing in this package (every function has at least one independent pin).
"""

from .scan import (  # noqa: F401
    softplus,
    silu,
    combine,
    discretise,
    scan_fwd,
    state_update,
    scan_pairs_blelloch,
    segment_aggregate,
    carry_combine,
)
from .scan_bwd import scan_bwd  # noqa: F401
from .conv1d import causal_conv1d, conv1d_update  # noqa: F401
from .block import mamba_block_fwd  # noqa: F401
