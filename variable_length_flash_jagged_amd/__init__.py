"""Jagged Flash Attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libjfa.so`` built from ``csrc/``; this package
is a thin ctypes binding over it (``binding.py``) plus the seeded input generators
(``workloads.py``) and the FLOP/byte accounting used by the benchmark
(``metrics.py``).  Importing the package loads nothing; the library is loaded on the
first call into the binding and a missing or stale build raises immediately.
"""

__all__ = ["binding", "workloads", "metrics"]
