"""CPU oracle for the ScoutAttention GPU-side decode path (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It is plain float64 NumPy and shares nothing with the HIP path.
"""
from .scout_oracle import *  # noqa: F401,F403
from .scout_oracle import Partial, PairResult  # noqa: F401
