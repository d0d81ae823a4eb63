"""Plain CPU oracle for group-wise int4 weight quantization and the W4A16 linear.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path never does.
"""
from .w4_oracle import *  # noqa: F401,F403
