"""Float64 CPU oracle for the rotated INT2 KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything under this directory; only the test suite, the smoke check and the
CPU-baseline leg of the benchmark do.  It shares no code with the HIP library.
"""
from .kvq_oracle import *  # noqa: F401,F403
