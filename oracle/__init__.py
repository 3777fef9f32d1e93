"""CPU oracle of the fused SO(2) convolution -- test infrastructure only.

Importable by the tests, the package's smoke check and the benchmark's CPU
baseline leg; never by the product path.
"""
from . import so2conv_oracle  # noqa: F401
