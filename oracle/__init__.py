"""CPU oracle for the two-stage retrieval head: test infrastructure only.

Imported only by tests, the package entry's smoke check and the benchmark's
CPU-baseline leg.  The library never imports it.
"""
from . import flashhead_ref  # noqa: F401
