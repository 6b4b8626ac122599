"""Python binding of libattn.so, the gfx950 fused exact-attention library.

The functions carry the C ABI's names and only marshal arguments: they check the torch
tensors' dtype, device, shape and layout, pass raw device pointers and the current HIP
stream to the library, and turn a nonzero status into :class:`AttnError`. Every step of
the computation runs in the library's HIP kernels; there is no CPU or PyTorch fallback, and
importing this package fails loudly when the library has not been built.

torch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "AttnError", "library_path", "load_library",
    "attn_fwd", "attn_fwd_f32", "attn_fwd_ex", "attn_fwd_workspace_bytes", "attn_fwd_force_mapping",
    "FWD_MAPPINGS", "attn_fwd_paged", "attn_fwd_paged_workspace_bytes", "attn_decode_paged",
    "attn_decode_paged_ex", "attn_decode_paged_full", "attn_decode_paged_noalloc",
    "attn_decode_noalloc_max_bytes", "attn_decode_workspace_bytes",
    "attn_decode_workspace_bytes_ex", "attn_decode_default_workers", "attn_status_string",
    "attn_last_error", "attn_release_workspace", "attn_abi_version", "attn_add_rms_norm",
    "add_rms_norm", "attn_rope_cache_write", "rope_cache_write", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")

# Every symbol include/attn.h declares, with its ctypes signature.
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGNATURES = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _Z, _P]),
    "attn_fwd_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "attn_fwd_force_mapping": (_I, [_I]),
    "attn_fwd_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                            _I, _I, _F, _P, _Z, _P]),
    "attn_fwd_paged_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "attn_decode_paged_ex": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _Z,
                                  _P]),
    "attn_decode_paged_full": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I,
                                    _I, _P, _Z, _P]),
    "attn_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F,
                                       _I, _I, _I, _P]),
    "attn_decode_noalloc_max_bytes": (_Z, []),
    "attn_decode_workspace_bytes": (_Z, [_I, _I, _I]),
    "attn_decode_workspace_bytes_ex": (_Z, [_I, _I, _I, _I, _I]),
    "attn_decode_default_workers": (_I, []),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_release_workspace": (None, []),
    "attn_abi_version": (_I, []),
    "attn_add_rms_norm": (_I, [_P, _P, _P, _P, _P, _I, _I, _F, _P]),
    "attn_rope_cache_write": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                   _I, _I, _F, _P]),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def _hip_runtimes_mapped():
    """Distinct libamdhip64 files mapped into this process (Linux only)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:
        return []


def load_library():
    """Load libattn.so once and attach the C signatures. Raises if it is not built.

    torch is imported first: its bundled HIP runtime has the same soname as the system one
    libattn.so was linked against, so the dynamic loader then binds libattn.so to the runtime
    torch already uses. Loading libattn.so first would put two HIP runtimes in the process,
    and the second one to initialise finds no device."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with `python exact_attention_42_amd/build.py` "
                "(there is no fallback implementation)")
        import torch  # noqa: F401  (binds the HIP runtime before libattn.so is loaded)
        lib = ctypes.CDLL(_LIB_PATH)
        rts = _hip_runtimes_mapped()
        if len(rts) > 1:
            raise ImportError(f"more than one HIP runtime is loaded in this process: {rts}")
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


load_library()


# ---------------------------------------------------------------------------------------
def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_last_error() -> str:
    return load_library().attn_last_error().decode()


def attn_abi_version() -> int:
    return load_library().attn_abi_version()


def attn_decode_default_workers() -> int:
    return load_library().attn_decode_default_workers()


def attn_decode_workspace_bytes(B: int, Hq: int, D: int) -> int:
    return load_library().attn_decode_workspace_bytes(B, Hq, D)


def attn_decode_workspace_bytes_ex(B: int, Hq: int, Hkv: int, D: int, num_workers: int = 0) -> int:
    return load_library().attn_decode_workspace_bytes_ex(B, Hq, Hkv, D, num_workers)


def attn_release_workspace() -> None:
    load_library().attn_release_workspace()


def _check(status: int) -> None:
    if status != 0:
        raise AttnError(status, f"{attn_status_string(status)}: {attn_last_error()}")


def _torch():
    import torch
    return torch


def _stream_ptr(device, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(stream.cuda_stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtype, device, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _fwd(fn_name, dtype, q, k, v, causal, scale, out, lse, want_lse, stream, workspace=None):
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != (B, Hkv, Sk, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dtype, dev)
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=dtype, device=dev)
    _need(out, "out", dtype, dev, (B, Hq, Sq, D))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, (B, Hq, Sq))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    fn = getattr(load_library(), fn_name)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, D,
            1 if causal else 0, float(scale)]
    if fn_name == "attn_fwd_ex":
        if workspace is not None:
            _need(workspace, "workspace", torch.uint8, dev)
        args += [_ptr(workspace), int(workspace.numel()) if workspace is not None else 0]
    with torch.cuda.device(dev):
        _check(fn(*args, _stream_ptr(dev, stream)))
    return out, lse


def attn_fwd(q, k, v, causal=False, scale=None, out=None, lse=None, want_lse=True, stream=None,
             workspace=None):
    """bf16 forward. q [B,Hq,Sq,D], k/v [B,Hkv,Sk,D] (bfloat16, contiguous, same GPU).

    Returns (out [B,Hq,Sq,D] bf16, lse [B,Hq,Sq] fp32 or None). ``scale`` defaults to
    1/sqrt(D). The work is enqueued on ``stream`` (default: torch's current stream).
    ``workspace`` is an optional uint8 device tensor of at least attn_fwd_workspace_bytes(...)
    bytes for the key-range splits of few-tile problems (None: the library's own)."""
    return _fwd("attn_fwd_ex", _torch().bfloat16, q, k, v, causal, scale, out, lse, want_lse,
                stream, workspace)


def attn_fwd_ex(*args, **kw):
    """Alias of :func:`attn_fwd` (which always goes through the C entry point attn_fwd_ex)."""
    return attn_fwd(*args, **kw)


def attn_fwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, causal) -> int:
    return load_library().attn_fwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, 1 if causal else 0)


FWD_MAPPINGS = {"tile": 0, "pair": 1, "wide": 2}


def attn_fwd_force_mapping(mapping) -> int:
    """Force the bf16 forward's work mapping ("tile", "pair", "wide" or its number; None or -1 =
    chosen per problem) for measurement and testing; returns the previous setting."""
    if mapping is None:
        mapping = -1
    elif isinstance(mapping, str):
        mapping = FWD_MAPPINGS[mapping]
    return load_library().attn_fwd_force_mapping(int(mapping))


def attn_fwd_f32(q, k, v, causal=False, scale=None, out=None, lse=None, want_lse=True,
                 stream=None):
    """fp32 forward; same contract as :func:`attn_fwd` with float32 q, k, v, out."""
    return _fwd("attn_fwd_f32", _torch().float32, q, k, v, causal, scale, out, lse, want_lse,
                stream)


def attn_fwd_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, ctx_lens, max_q, max_ctx,
                   causal=True, scale=None, out=None, lse=None, want_lse=True,
                   check_blocks=True, workspace=None, stream=None):
    """Prefill of packed query tokens against a paged KV cache (bf16); returns (out, lse).

    q [T, Hq, D]; k_cache, v_cache [num_blocks, Hkv, 16, D]; block_table [B, stride] int32;
    cu_seqlens_q [B + 1] int32 (sequence b's tokens are rows cu[b] .. cu[b+1]-1 of q);
    ctx_lens [B] int32 (each sequence's keys, its new tokens included). ``max_q`` and
    ``max_ctx`` bound the per-sequence query and key counts (host integers: no
    synchronisation). The table's row stride is passed as ``block_table.shape[1]``;
    ``check_blocks`` passes the pool size so out-of-pool entries mask their keys instead of
    being read. ``workspace``: optional uint8 device tensor of at least
    attn_fwd_paged_workspace_bytes(...) bytes (None: the library's own)."""
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [T, Hq, D] and caches [num_blocks, Hkv, block_size, D]")
    T, Hq, D = q.shape
    nb, Hkv, bs, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [B, stride]")
    B = block_table.shape[0]
    _need(block_table, "block_table", torch.int32, dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev, (B + 1,))
    _need(ctx_lens, "ctx_lens", torch.int32, dev, (B,))
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev, (T, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, (T, Hq))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(dev):
        _check(load_library().attn_fwd_paged(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(cu_seqlens_q),
            _ptr(ctx_lens), _ptr(out), _ptr(lse), B, T, Hq, Hkv, D, bs, int(max_q),
            int(max_ctx), int(block_table.shape[1]), int(nb) if check_blocks else 0,
            1 if causal else 0, float(scale), _ptr(workspace),
            int(workspace.numel()) if workspace is not None else 0, _stream_ptr(dev, stream)))
    return out, lse


def attn_fwd_paged_workspace_bytes(B, T, Hq, Hkv, D, max_q, max_ctx, causal=True) -> int:
    return load_library().attn_fwd_paged_workspace_bytes(B, T, Hq, Hkv, D, max_q, max_ctx,
                                                         1 if causal else 0)


def _decode_checks(q, k_cache, v_cache, block_table, ctx_lens):
    torch = _torch()
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and caches [num_blocks, Hkv, block_size, D]")
    B, Hq, D = q.shape
    nb, Hkv, bs, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes do not match q")
    dev = q.device
    _need(q, "q", torch.bfloat16, dev)
    _need(k_cache, "k_cache", torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev)
    _need(ctx_lens, "ctx_lens", torch.int32, dev, (B,))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, stride]")
    _need(block_table, "block_table", torch.int32, dev)
    return B, Hq, D, nb, Hkv, bs, dev


def attn_decode_paged(q, k_cache, v_cache, block_table, ctx_lens, scale=None, out=None,
                      stream=None):
    """Paged one-token decode (bf16); returns out [B, Hq, D].

    Goes through the C entry point attn_decode_paged_full with the block table's actual row
    stride (``block_table.shape[1]``, which may exceed the longest context's block count, as
    in a table preallocated for the maximum context) and the pool size ``k_cache.shape[0]``,
    so a table entry outside the pool is skipped instead of read. (The 13-argument C entry
    point attn_decode_paged derives the stride from ctx_lens instead.)"""
    o, _ = attn_decode_paged_full(q, k_cache, v_cache, block_table, ctx_lens, scale=scale,
                                  out=out, want_lse=False, stream=stream)
    return o


def attn_decode_paged_ex(q, k_cache, v_cache, block_table, ctx_lens, scale=None, out=None,
                         workspace=None, stream=None):
    """The C entry point attn_decode_paged_ex: the block table's row stride passed explicitly
    (``block_table.shape[1]``) and an optional caller workspace (a uint8 device tensor of at
    least attn_decode_workspace_bytes(B, Hq, D) bytes; None = the library's own). Block ids
    are not range-checked; returns out [B, Hq, D]."""
    torch = _torch()
    B, Hq, D, nb, Hkv, bs, dev = _decode_checks(q, k_cache, v_cache, block_table, ctx_lens)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev, (B, Hq, D))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(dev):
        _check(load_library().attn_decode_paged_ex(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), _ptr(out),
            B, Hq, Hkv, D, bs, float(scale), int(block_table.shape[1]), _ptr(workspace),
            int(workspace.numel()) if workspace is not None else 0, _stream_ptr(dev, stream)))
    return out


def attn_decode_paged_full(q, k_cache, v_cache, block_table, ctx_lens, scale=None, out=None,
                         lse=None, want_lse=True, check_blocks=True, num_workers=0,
                         workspace=None, stream=None):
    """Paged decode with the explicit controls of the C ABI: returns (out, lse). The row
    stride of ``block_table`` is passed explicitly; ``check_blocks`` passes the pool size so
    out-of-range entries are skipped instead of read; ``workspace`` is an optional uint8
    device tensor of at least attn_decode_workspace_bytes_ex(B, Hq, Hkv, D, num_workers) bytes;
    ``num_workers`` sets how many worker waves split the blocks (0 = the device default)."""
    torch = _torch()
    B, Hq, D, nb, Hkv, bs, dev = _decode_checks(q, k_cache, v_cache, block_table, ctx_lens)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev, (B, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, (B, Hq))
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(dev):
        _check(load_library().attn_decode_paged_full(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), _ptr(out),
            _ptr(lse), B, Hq, Hkv, D, bs, float(scale), int(block_table.shape[1]),
            int(nb) if check_blocks else 0, int(num_workers), _ptr(workspace),
            int(workspace.numel()) if workspace is not None else 0, _stream_ptr(dev, stream)))
    return out, lse


def attn_decode_noalloc_max_bytes() -> int:
    return load_library().attn_decode_noalloc_max_bytes()


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, ctx_lens, scale=None, out=None,
                              lse=None, want_lse=True, check_blocks=True, num_workers=0,
                              stream=None):
    """Paged decode whose partial results live in the library's fixed device array (the C
    entry point allocates nothing; ``out``/``lse`` are allocated here only when not given).
    Returns (out, lse). Calls that overlap on one device race on that array."""
    torch = _torch()
    B, Hq, D, nb, Hkv, bs, dev = _decode_checks(q, k_cache, v_cache, block_table, ctx_lens)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, dev, (B, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, (B, Hq))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    with torch.cuda.device(dev):
        _check(load_library().attn_decode_paged_noalloc(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), _ptr(out),
            _ptr(lse), B, Hq, Hkv, D, bs, float(scale), int(block_table.shape[1]),
            int(nb) if check_blocks else 0, int(num_workers), _stream_ptr(dev, stream)))
    return out, lse


def add_rms_norm(x, residual, weight, eps=1e-6, out=None, residual_out=None, stream=None):
    """Fused residual add + RMS norm (bf16): returns (out, residual_out) with
    residual_out = x + residual and out = residual_out * rsqrt(mean(residual_out^2) + eps) *
    weight over the last dimension. x and residual are [..., d], weight [d]. Pass out=x and/or
    residual_out=residual to work in place."""
    torch = _torch()
    if x.dim() < 1 or tuple(residual.shape) != tuple(x.shape):
        raise ValueError(f"x {tuple(x.shape)} and residual {tuple(residual.shape)} must match")
    d = x.shape[-1]
    M = x.numel() // d if d else 0
    dev = x.device
    _need(x, "x", torch.bfloat16, dev)
    _need(residual, "residual", torch.bfloat16, dev)
    _need(weight, "weight", torch.bfloat16, dev, (d,))
    if out is None:
        out = torch.empty_like(x)
    if residual_out is None:
        residual_out = torch.empty_like(x)
    _need(out, "out", torch.bfloat16, dev, tuple(x.shape))
    _need(residual_out, "residual_out", torch.bfloat16, dev, tuple(x.shape))
    with torch.cuda.device(dev):
        _check(load_library().attn_add_rms_norm(
            _ptr(x), _ptr(residual), _ptr(weight), _ptr(out), _ptr(residual_out), int(M), int(d),
            float(eps), _stream_ptr(dev, stream)))
    return out, residual_out


def attn_add_rms_norm(*args, **kw):
    """Alias of :func:`add_rms_norm` under the C symbol's name."""
    return add_rms_norm(*args, **kw)


def rope_cache_write(q, k, v, positions, k_cache, v_cache, block_table, seq_ids=None,
                     base=10000.0, q_out=None, check_blocks=True, stream=None):
    """Rotary embedding of q [T, Hq, D] and k [T, Hkv, D] at int32 ``positions`` [T], and the
    store of the rotated keys and the values into the paged caches [num_blocks, Hkv, 16, D]
    through ``block_table`` [num_seqs, stride] (token t belongs to sequence ``seq_ids[t]``,
    or to sequence t when ``seq_ids`` is None). Returns the rotated queries (``q_out``, which
    may be ``q``). ``check_blocks`` passes the pool size so out-of-range entries store
    nothing."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q and k must be [T, H, D] and the caches [num_blocks, Hkv, 16, D]")
    T, Hq, D = q.shape
    nb, Hkv, bs, Dc = k_cache.shape
    if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D) or Dc != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)} cache{tuple(k_cache.shape)}")
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, torch.bfloat16, dev)
    _need(v_cache, "v_cache", torch.bfloat16, dev, tuple(k_cache.shape))
    _need(positions, "positions", torch.int32, dev, (T,))
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, stride]")
    _need(block_table, "block_table", torch.int32, dev)
    if seq_ids is not None:
        _need(seq_ids, "seq_ids", torch.int32, dev, (T,))
    if q_out is None:
        q_out = torch.empty_like(q)
    _need(q_out, "q_out", torch.bfloat16, dev, (T, Hq, D))
    with torch.cuda.device(dev):
        _check(load_library().attn_rope_cache_write(
            _ptr(q), _ptr(k), _ptr(v), _ptr(q_out), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), _ptr(positions), _ptr(seq_ids), int(T),
            int(block_table.shape[0]), int(Hq), int(Hkv), int(D), int(bs),
            int(block_table.shape[1]), int(nb) if check_blocks else 0, float(base),
            _stream_ptr(dev, stream)))
    return q_out


def attn_rope_cache_write(*args, **kw):
    """Alias of :func:`rope_cache_write` under the C symbol's name."""
    return rope_cache_write(*args, **kw)
