"""fp64 CPU reference for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package's ``smoke()`` check and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the HIP library.

Modules:
  attention  forward, backward, split-KV decode and combine (plain definitions)
  fp8        e4m3 codec, per-block quantiser, Hadamard rotation
  schedule   greedy list scheduling for the longest-first tile order
"""
from . import attention, fp8, schedule  # noqa: F401
