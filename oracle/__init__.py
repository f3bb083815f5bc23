"""CPU oracle for selective sparse attention.

Test infrastructure only: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library's product path never does.
"""
from .spattn_oracle import *  # noqa: F401,F403
