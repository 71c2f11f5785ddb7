"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package holds no attention, softmax, quantisation or write arithmetic:
only lengths, block allocation, random values and the caller-side slot
assignment that an engine performs before launching the write.
"""

from .configs import (  # noqa: F401
    Step,
    VarlenContig,
    build_step,
    config,
    config_names,
    page2_varlen_example,
    random_varlen_contig,
)
