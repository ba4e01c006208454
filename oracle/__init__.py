"""CPU oracle for the product-VQ KV-cache hot path (test infrastructure only).

Only the test suite, the smoke check of the entry script and the CPU-baseline
leg of the benchmark may import this package.  It shares no code with the HIP
library and imports nothing from it.
"""
from .vq_oracle import *  # noqa: F401,F403
