"""fp64 CPU oracle of the FLARE / FLARE++ routing forward (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the GPU product path never imports it.
"""
from .oracle import *  # noqa: F401,F403
