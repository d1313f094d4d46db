"""CPU oracle for the SVDQuant W4A4 + low-rank linear and the W4A16 projection.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package. The product path never routes
through it, and it shares no code with the GPU library or its Python binding.
"""
from .svdq_oracle import *  # noqa: F401,F403
