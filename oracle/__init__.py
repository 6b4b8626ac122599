"""CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. The library path (the HIP kernels behind the C ABI and their
Python binding) never imports, calls or falls back to it.

See ``oracle/direct.py`` for what is computed and which passage each function follows.
"""
from .direct import attention, attention_rows, decode_paged, gather_paged

__all__ = ["attention", "attention_rows", "decode_paged", "gather_paged"]
