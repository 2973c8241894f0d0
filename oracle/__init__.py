"""CPU oracle for draft-block verification (test infrastructure only).

Importable by the test suite, the smoke check and the benchmark's CPU
baseline leg; nothing in the product library uses it.
"""
from . import sd_oracle  # noqa: F401
