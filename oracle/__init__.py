"""CPU oracle for exact attention, the fused residual-add RMS norm and the RoPE + paged-cache
write -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. The library path (the HIP kernels behind the C ABI and their
Python binding) never imports, calls or falls back to it.

See ``oracle/direct.py`` (attention), ``oracle/rmsnorm.py`` (add_rms_norm) and
``oracle/rotary.py`` (rotary embedding + cache write) for what is computed and which passage
each function follows.
"""
from .direct import attention, attention_rows, decode_paged, gather_paged, prefill_paged
from .rmsnorm import add_rms_norm
from .rotary import rope, rope_cache_write

__all__ = ["attention", "attention_rows", "decode_paged", "gather_paged", "add_rms_norm",
           "rope", "rope_cache_write"]
