"""CPU oracle for MLA / GQLA decode over a compressed latent cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this package: only the
test suite, the smoke check and the bench's CPU-baseline leg use it. It shares no code with
the HIP library and never reads anything the GPU produced.
"""
from .mla_oracle import *  # noqa: F401,F403
