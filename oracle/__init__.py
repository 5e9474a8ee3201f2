"""Plain CPU oracle for the block-scaled FP4 expert MLP.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package. The GPU library never calls it,
and it shares no code, tables or helpers with the GPU library.

See ``oracle/mx_oracle.py`` for the functions and the passages they follow.
"""

from .mx_oracle import *  # noqa: F401,F403
