"""CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP library never does.  See ``oracle.rownorm``.
"""

from .rownorm import *  # noqa: F401,F403
from .rownorm import __all__  # noqa: F401
