"""fp64 CPU oracle for the KDA forward prefill (test infrastructure only).

Importable only by the tests, the package smoke check and the benchmark's
CPU-baseline leg.  The library never imports it.
"""
from .kda_oracle import *  # noqa: F401,F403
