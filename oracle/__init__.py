"""CPU oracle for the IsoQuant packed 3-bit KV cache -- test infrastructure only.

Imported by the tests, the smoke entry point and the benchmark's CPU-baseline
leg; never by the product path. See ``oracle.iqref`` for the definitions.
"""
from . import iqref  # noqa: F401
