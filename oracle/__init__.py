"""CPU oracle for the fused quantized linear layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never do.
"""
from .oracle import *  # noqa: F401,F403
