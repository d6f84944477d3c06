"""CPU oracle for MLA latent-KV decode (fp64 numpy).

TEST INFRASTRUCTURE: imported only by the tests, the package smoke check and
the benchmark's CPU-baseline leg.  The product path never imports it.
"""
from .mla_oracle import *  # noqa: F401,F403
from . import mla_oracle  # noqa: F401
