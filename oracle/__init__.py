"""TEST INFRASTRUCTURE ONLY: the CPU oracle for the NF4-LoRA linear layer.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.
"""
from .oracle import *  # noqa: F401,F403
