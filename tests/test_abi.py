"""The C-ABI library on the host: it loads, exports every symbol the header declares, and
rejects bad arguments with the documented status codes before launching anything (these
calls never reach the GPU, so they run without one)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_42_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, SCALE, HIP, NOMEM, WS = range(9)
P = 0x10000          # a fake, 16-byte aligned device address: never dereferenced here
NAN = float("nan")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_what_the_binding_wraps():
    assert header_functions() == sorted(A.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = A.load_library()
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", A.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)$", out, flags=re.M))
    assert set(header_functions()) <= exported


def test_status_strings_and_version():
    for code in range(9):
        assert A.attn_status_string(code) not in ("", "unknown status")
    assert A.attn_status_string(99) == "unknown status"
    assert A.attn_abi_version() == 10


def fwd(*, q=P, k=P, v=P, o=P, lse=0, B=1, Hq=32, Hkv=8, Sq=128, Sk=128, D=128, causal=1,
        scale=0.08, f32=False):
    lib = A.load_library()
    fn = lib.attn_fwd_f32 if f32 else lib.attn_fwd
    return fn(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, None)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(o=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL),
    (dict(B=-1), SHAPE), (dict(Sq=-3), SHAPE), (dict(Sk=-1), SHAPE), (dict(Hq=0), SHAPE),
    (dict(Hkv=0), SHAPE), (dict(Hq=32, Hkv=6), SHAPE), (dict(D=96), UNSUP), (dict(D=256), UNSUP),
    (dict(q=P + 8), ALIGN), (dict(k=P + 2), ALIGN), (dict(v=P + 4), ALIGN), (dict(o=P + 1), ALIGN),
    (dict(lse=P + 2), ALIGN), (dict(scale=NAN), SCALE), (dict(scale=float("inf")), SCALE),
    (dict(scale=-0.1), SCALE), (dict(B=70000, Hq=40000, Hkv=1), SHAPE),
])
def test_fwd_rejects(kw, code, f32):
    assert fwd(f32=f32, **kw) == code
    assert A.attn_last_error() != ""


def test_fwd_bf16_rejects_a_head_over_2gib():
    # one head's K must fit the kernel's 32-bit buffer offsets; the f32 path has no such limit
    assert fwd(Sk=1 << 23, D=128) == SHAPE
    assert "2^31" in A.attn_last_error()
    assert fwd(Sk=1 << 24, D=64) == SHAPE


@pytest.mark.parametrize("kw", [dict(B=0), dict(Sq=0), dict(B=0, q=0, k=0, v=0, o=0),
                                dict(Sq=0, q=0, o=0)])
def test_fwd_empty_problem_is_a_no_op(kw):
    assert fwd(**kw) == OK
    assert A.attn_last_error() == ""


def fwdp(*, q=P, kc=P, vc=P, table=P, cu=P, ctx=P, o=P, lse=0, B=1, T=512, Hq=32, Hkv=8, D=128,
         bs=16, max_q=512, max_ctx=4096, stride=256, nblocks=0, causal=1, scale=0.08, ws=P,
         ws_bytes=1 << 40):
    return A.load_library().attn_fwd_paged(q, kc, vc, table, cu, ctx, o, lse, B, T, Hq, Hkv, D,
                                           bs, max_q, max_ctx, stride, nblocks, causal, scale,
                                           ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(kc=0), NULL), (dict(vc=0), NULL), (dict(table=0), NULL),
    (dict(cu=0), NULL), (dict(ctx=0), NULL), (dict(o=0), NULL), (dict(B=-1), SHAPE),
    (dict(T=-1), SHAPE), (dict(max_q=-1), SHAPE), (dict(max_ctx=-2), SHAPE), (dict(Hq=0), SHAPE),
    (dict(Hq=32, Hkv=5), SHAPE), (dict(stride=0), SHAPE), (dict(T=1 << 27, Hq=32), SHAPE),
    (dict(B=1 << 20, stride=1 << 12), SHAPE), (dict(D=96), UNSUP), (dict(bs=32), UNSUP),
    (dict(q=P + 8), ALIGN), (dict(kc=P + 4), ALIGN), (dict(vc=P + 2), ALIGN),
    (dict(o=P + 2), ALIGN), (dict(table=P + 2), ALIGN), (dict(cu=P + 1), ALIGN),
    (dict(ctx=P + 2), ALIGN), (dict(lse=P + 2), ALIGN), (dict(scale=NAN), SCALE),
    (dict(scale=-1.0), SCALE), (dict(ws_bytes=100), WS), (dict(ws=P + 4), WS),
])
def test_fwd_paged_rejects(kw, code):
    # (the default shape, a 512-token chunk over a 4096-token context, splits its keys, so the
    #  workspace checks run too)
    assert fwdp(**kw) == code
    assert A.attn_last_error() != ""


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(max_q=0),
                                dict(B=0, q=0, kc=0, vc=0, table=0, cu=0, ctx=0, o=0)])
def test_fwd_paged_empty_problem_is_a_no_op(kw):
    assert fwdp(**kw) == OK
    assert A.attn_last_error() == ""


def test_fwd_paged_workspace_size():
    # 128 query tiles on 256 CUs: ceil(2 * 256 / 128) = 4 key ranges per tile, each of the
    # T * Hq rows with D bf16 outputs and 2 floats (max, sum) per range
    if A.attn_fwd_paged_workspace_bytes(1, 512, 32, 8, 128, 512, 4096, 1) == 0:
        pytest.skip("device reports other than 256 CUs")
    assert A.attn_fwd_paged_workspace_bytes(1, 512, 32, 8, 128, 512, 4096, 1) == \
        4 * 512 * 32 * (128 * 2 + 2 * 4)
    # enough query tiles: no splits
    assert A.attn_fwd_paged_workspace_bytes(8, 32768, 32, 8, 128, 4096, 4096, 1) == 0
    for bad in [(-1, 1, 1, 1, 64, 1, 1, 1), (1, 1, 6, 4, 64, 1, 1, 1), (1, 1, 1, 1, 80, 1, 1, 1),
                (1, 1, 1, 1, 64, -1, 1, 1)]:
        assert A.attn_fwd_paged_workspace_bytes(*bad) == 0, bad
    need = A.attn_fwd_paged_workspace_bytes(1, 512, 32, 8, 128, 512, 4096, 1)
    assert fwdp(ws_bytes=need - 1) == WS


def dec(*, q=P, kc=P, vc=P, table=P, ctx=P, o=P, lse=0, B=64, Hq=32, Hkv=8, D=128, bs=16,
        scale=0.08, stride=0, nblocks=0, workers=0, ws=P, ws_bytes=1 << 40, ex=True):
    lib = A.load_library()
    if not ex:
        return lib.attn_decode_paged(q, kc, vc, table, ctx, o, B, Hq, Hkv, D, bs, scale, None)
    return lib.attn_decode_paged_full(q, kc, vc, table, ctx, o, lse, B, Hq, Hkv, D, bs, scale,
                                    stride, nblocks, workers, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(kc=0), NULL), (dict(vc=0), NULL), (dict(table=0), NULL),
    (dict(ctx=0), NULL), (dict(o=0), NULL), (dict(B=-1), SHAPE), (dict(Hq=0), SHAPE),
    (dict(Hq=32, Hkv=5), SHAPE), (dict(Hq=64, Hkv=2), UNSUP), (dict(D=80), UNSUP),
    (dict(bs=32), UNSUP), (dict(bs=8), UNSUP), (dict(q=P + 8), ALIGN), (dict(kc=P + 4), ALIGN),
    (dict(o=P + 2), ALIGN), (dict(table=P + 2), ALIGN), (dict(ctx=P + 1), ALIGN),
    (dict(lse=P + 2), ALIGN), (dict(scale=NAN), SCALE), (dict(scale=-1.0), SCALE),
    (dict(workers=65537), SHAPE), (dict(workers=-1), SHAPE), (dict(ws_bytes=100), WS),
    (dict(ws=P + 4), WS), (dict(B=70000), SHAPE),
])
def test_decode_rejects(kw, code):
    assert dec(**kw) == code
    assert A.attn_last_error() != ""


def dec_contract(*, q=P, kc=P, vc=P, table=P, ctx=P, o=P, B=64, Hq=32, Hkv=8, D=128, bs=16,
                 scale=0.08, stride=0, ws=P, ws_bytes=1 << 40):
    return A.load_library().attn_decode_paged_ex(q, kc, vc, table, ctx, o, B, Hq, Hkv, D, bs,
                                                 scale, stride, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(table=0), NULL), (dict(o=0), NULL), (dict(B=-1), SHAPE),
    (dict(Hq=32, Hkv=5), SHAPE), (dict(Hq=64, Hkv=2), UNSUP), (dict(D=80), UNSUP),
    (dict(bs=8), UNSUP), (dict(kc=P + 4), ALIGN), (dict(ctx=P + 1), ALIGN),
    (dict(scale=NAN), SCALE), (dict(ws_bytes=100), WS), (dict(ws=P + 4), WS),
])
def test_decode_contract_entry_point_rejects(kw, code):
    # the contract form of attn_decode_paged_ex: explicit stride and caller workspace only
    assert dec_contract(**kw) == code
    assert A.attn_last_error() != ""


def test_decode_contract_workspace_bound():
    # attn_decode_workspace_bytes(B, Hq, D) covers every Hkv the decode accepts for Hq
    for B, Hq, D in [(64, 32, 128), (3, 12, 64), (1, 1, 64), (5, 48, 128), (0, 8, 64)]:
        need = A.attn_decode_workspace_bytes(B, Hq, D)
        ok = [h for h in range(1, Hq + 1) if Hq % h == 0 and Hq // h <= 16]
        assert ok and need == max(A.attn_decode_workspace_bytes_ex(B, Hq, h, D, 0) for h in ok)
    assert A.attn_decode_workspace_bytes(1, 4, 80) == 0
    assert A.attn_decode_workspace_bytes(-1, 4, 64) == 0
    # one byte short of the need of the Hkv that needs most is refused before any launch
    h_max = max((h for h in range(1, 33) if 32 % h == 0 and 32 // h <= 16),
                key=lambda h: A.attn_decode_workspace_bytes_ex(64, 32, h, 128, 0))
    assert dec_contract(ws_bytes=A.attn_decode_workspace_bytes(64, 32, 128) - 1, Hkv=h_max) == WS


def test_decode_plain_entry_point_rejects_before_launch():
    assert dec(ex=False, q=0) == NULL
    assert dec(ex=False, bs=32) == UNSUP
    assert dec(ex=False, B=0) == OK


def test_decode_default_workers():
    w = A.attn_decode_default_workers()
    assert 1 <= w <= 65536
    if "ATTN_DECODE_WORKERS" not in os.environ:
        assert w % 3 == 0       # three worker waves per compute unit


def ws_bytes(B, Hq, Hkv, D, W):
    g = Hq // Hkv
    head = (W + B * Hkv) * g * (D + 2) * 4
    return (head + 15) // 16 * 16 + B * Hkv * 2 * 4


def test_decode_workspace_size():
    w = A.attn_decode_default_workers()
    assert A.attn_decode_workspace_bytes_ex(64, 32, 8, 128, 0) == ws_bytes(64, 32, 8, 128, w)
    assert A.attn_decode_workspace_bytes_ex(3, 5, 5, 64, 7) == ws_bytes(3, 5, 5, 64, 7)
    assert A.attn_decode_workspace_bytes_ex(3, 6, 2, 64, 1) == ws_bytes(3, 6, 2, 64, 1)
    assert A.attn_decode_workspace_bytes_ex(0, 32, 8, 128, 5) == ws_bytes(0, 32, 8, 128, 5)
    for bad in [(1, 1, 1, 64, 65537), (1, 1, 1, 64, -1), (1, 6, 4, 64, 1), (1, 1, 1, 80, 1),
                (-1, 1, 1, 64, 1), (1, 34, 2, 64, 1), (70000, 1, 1, 64, 1)]:
        assert A.attn_decode_workspace_bytes_ex(*bad) == 0, bad
    # one byte less than the reported size is refused before anything is launched
    need = A.attn_decode_workspace_bytes_ex(64, 32, 8, 128, 4)
    assert dec(workers=4, ws_bytes=need - 1) == WS


def noalloc(*, q=P, kc=P, vc=P, table=P, ctx=P, o=P, lse=0, B=64, Hq=32, Hkv=8, D=128, bs=16,
            scale=0.08, stride=256, nblocks=0, workers=768):
    return A.load_library().attn_decode_paged_noalloc(q, kc, vc, table, ctx, o, lse, B, Hq, Hkv,
                                                      D, bs, scale, stride, nblocks, workers,
                                                      None)


def test_decode_noalloc_checks_before_anything_else():
    """The allocation-free decode validates like the _ex entry point and refuses a problem
    whose partial results do not fit its fixed array, all before touching the device."""
    cap = A.attn_decode_noalloc_max_bytes()
    assert cap == 8 << 20
    assert noalloc(q=0) == NULL
    assert noalloc(bs=32) == UNSUP
    assert noalloc(kc=P + 2) == ALIGN
    assert noalloc(scale=NAN) == SCALE
    assert noalloc(Hq=33) == SHAPE
    assert noalloc(B=0) == OK
    # the largest batch at 768 workers that fits, and the next one that does not
    fits = max(b for b in range(1, 4096) if ws_bytes(b, 32, 8, 128, 768) <= cap)
    assert noalloc(B=fits + 1) == WS
    assert "fixed scratch" in A.attn_last_error()
    assert noalloc(B=1, workers=65536) == WS     # too many worker slots


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        A.attn_fwd(x, x, x)


def test_one_hip_runtime_in_process():
    """libattn.so must share torch's HIP runtime (same soname); two runtimes in one process
    leave the second one without a device."""
    assert len(A._hip_runtimes_mapped()) <= 1


def test_library_defines_every_kernel_launch_stub():
    """A kernel whose host-side launch stub is missing makes the library fail to load with an
    undefined symbol; catch that at build time rather than on the GPU."""
    out = subprocess.run(["nm", "-D", A.library_path()], capture_output=True, text=True,
                         check=True).stdout
    undefined = [l for l in out.splitlines() if " U " in l and "device_stub" in l]
    assert undefined == []


def test_check_build_exports_the_same_symbols():
    """libattn_poison.so, the LDS-poisoning check build that the GPU tests compare with
    libattn.so, is built beside it from the same sources: it exports every declared symbol and
    misses no kernel launch stub."""
    path = os.path.join(os.path.dirname(A.library_path()), "libattn_poison.so")
    assert os.path.exists(path), f"{path} is missing: run __graft_entry__.build()"
    out = subprocess.run(["nm", "-D", path], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)$", out, flags=re.M))
    assert set(header_functions()) <= exported
    assert [l for l in out.splitlines() if " U " in l and "device_stub" in l] == []


def norm(*, x=P, r=P, w=P, o=P, t=P, M=4, d=4096, eps=1e-6):
    return A.load_library().attn_add_rms_norm(x, r, w, o, t, M, d, eps, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), NULL), (dict(r=0), NULL), (dict(w=0), NULL), (dict(o=0), NULL),
    (dict(t=0), NULL), (dict(M=-1), SHAPE), (dict(d=-8), SHAPE), (dict(d=0), UNSUP),
    (dict(d=12), UNSUP), (dict(d=65544), UNSUP), (dict(eps=NAN), SCALE),
    (dict(eps=-1e-6), SCALE), (dict(eps=float("inf")), SCALE), (dict(x=P + 8), ALIGN),
    (dict(t=P + 2), ALIGN), (dict(w=P + 4), ALIGN),
])
def test_norm_rejects(kw, code):
    assert norm(**kw) == code
    assert A.attn_last_error() != ""


def test_norm_empty_is_a_no_op():
    assert norm(M=0, x=0, r=0, w=0, o=0, t=0) == OK
    assert A.attn_last_error() == ""


def test_norm_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    x = torch.zeros(2, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        A.add_rms_norm(x, x, torch.zeros(16, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="must match"):
        A.add_rms_norm(x, torch.zeros(2, 8, dtype=torch.bfloat16), x[0])


def rope(*, q=P, k=P, v=P, qo=P, kc=P, vc=P, table=P, pos=P, seq=0, T=4, nseq=4, Hq=32, Hkv=8,
         D=128, bs=16, stride=8, nblocks=0, base=10000.0):
    return A.load_library().attn_rope_cache_write(q, k, v, qo, kc, vc, table, pos, seq, T, nseq,
                                                   Hq, Hkv, D, bs, stride, nblocks, base, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(qo=0), NULL),
    (dict(kc=0), NULL), (dict(vc=0), NULL), (dict(table=0), NULL), (dict(pos=0), NULL),
    (dict(T=-1), SHAPE), (dict(nseq=-1), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=0), SHAPE),
    (dict(stride=0), SHAPE), (dict(T=5, nseq=4), SHAPE), (dict(D=96), UNSUP),
    (dict(bs=32), UNSUP), (dict(base=NAN), SCALE), (dict(base=0.0), SCALE),
    (dict(base=-2.0), SCALE), (dict(q=P + 8), ALIGN), (dict(vc=P + 2), ALIGN),
    (dict(pos=P + 2), ALIGN), (dict(seq=P + 1), ALIGN),
])
def test_rope_rejects(kw, code):
    assert rope(**kw) == code
    assert A.attn_last_error() != ""


def test_rope_empty_and_sequence_map():
    assert rope(T=0, q=0, k=0, v=0, qo=0, kc=0, vc=0, table=0, pos=0) == OK
    # with a sequence map, more tokens than table rows is fine (the check is per token)
    assert rope(T=9, nseq=4, seq=P, q=0) == NULL


def test_fwd_ex_workspace_checks():
    lib = A.load_library()
    need = A.attn_fwd_workspace_bytes(1, 32, 8, 512, 4096, 128, True)
    # a 512-query chunk over 4096 keys has 128 query tiles: its key ranges are split
    assert need > 0
    assert A.attn_fwd_workspace_bytes(1, 32, 8, 2048, 2048, 128, True) == 0
    assert A.attn_fwd_workspace_bytes(1, 32, 8, 512, 4096, 96, True) == 0
    args = (P, P, P, P, 0, 1, 32, 8, 512, 4096, 128, 1, 0.08)
    assert lib.attn_fwd_ex(*args, P, need - 1, None) == WS
    assert lib.attn_fwd_ex(*args, P + 8, need, None) == WS
    assert lib.attn_fwd_ex(P, P, P, P, 0, 1, 32, 8, 512, 4096, 96, 1, 0.08, P, need,
                           None) == UNSUP
