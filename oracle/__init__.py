"""CPU oracle for exact attention and the fused residual-add RMS norm -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. The library path (the HIP kernels behind the C ABI and their
Python binding) never imports, calls or falls back to it.

See ``oracle/direct.py`` (attention) and ``oracle/rmsnorm.py`` (add_rms_norm) for what is
computed and which passage each function follows.
"""
from .direct import attention, attention_rows, decode_paged, gather_paged
from .rmsnorm import add_rms_norm

__all__ = ["attention", "attention_rows", "decode_paged", "gather_paged", "add_rms_norm"]
