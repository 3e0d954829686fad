"""CPU oracle for TT-EmbeddingBag -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and the
oracle imports nothing from the product package.
"""
from .tt_oracle import *  # noqa: F401,F403
