"""CPU oracle for the SmoothQuant W8A8 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, the smoke check and the CPU-baseline leg of the benchmark use
it. It shares no code with the HIP library (no kernels, headers, helpers or
tables) and imports nothing from it.
"""
from .smoothquant_oracle import *  # noqa: F401,F403
from .smoothquant_oracle import __all__  # noqa: F401
