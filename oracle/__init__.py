"""Float64 CPU oracle for Orthros attention — TEST INFRASTRUCTURE.

Imported only by the tests, the package smoke check and the benchmark's CPU-baseline leg.
It shares no code with the HIP path and imports nothing from it.

Parity pinning: every function here is pinned by CPU tests against something other than
itself (a library attention routine, closed forms, a hand-derived worked example and
invariants of the equations); no function is "parity unpinned".
"""
from .orthros_oracle import *  # noqa: F401,F403
from .orthros_oracle import __all__  # noqa: F401
