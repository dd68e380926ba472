"""CPU oracle for draft-block verification and foresight outcome scoring.

TEST INFRASTRUCTURE -- not part of the product.  Only tests/, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py may import, call or run
anything in this package.  It shares no code with the HIP library.

Modules:
  philox     -- Philox4x32-10 from its published definition (pinned to the
                published known-answer values).
  reference  -- RMSNorm, LM head, softmax at T, the acceptance rule, the bonus
                draw, the outcome law and top-N, all in float64.
Every function is pinned by a `-m "not gpu"` test in tests/test_oracle_*.py;
no function is left "parity unpinned".
"""
from . import philox, reference  # noqa: F401
from .reference import *  # noqa: F401,F403
