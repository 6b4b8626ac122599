"""The allocation-free paged decode (attn_decode_paged_noalloc, partial results in the library's
fixed device array) called through the C ABI, against attn_decode_paged_full with a caller
workspace (same kernels: the results must be identical bit for bit) and against the fp64
oracle, on two calls in a row where the second is smaller; the first call's partial results
are still in the array when the second runs."""
import ctypes

import numpy as np
import pytest
import torch

import exact_attention_42_amd as A
import oracle
import workloads as W
from tests.parity import check_bf16, check_lse, to_np

pytestmark = pytest.mark.gpu


def _upload(d, dev):
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return bf(d.q), bf(d.k_cache), bf(d.v_cache), i32(d.block_table), i32(d.ctx_lens)


def _c_noalloc(q, kc, vc, bt, ctx, o, lse, scale, workers):
    B, Hq, D = q.shape
    nb, Hkv = kc.shape[0], kc.shape[1]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = A.load_library().attn_decode_paged_noalloc(
        p(q), p(kc), p(vc), p(bt), p(ctx), p(o), p(lse), B, Hq, Hkv, D, 16, scale,
        int(bt.shape[1]), nb, workers, stream)
    assert rc == 0, A.attn_last_error()


def _c_ex(q, kc, vc, bt, ctx, o, lse, scale, workers):
    B, Hq, D = q.shape
    nb, Hkv = kc.shape[0], kc.shape[1]
    need = A.attn_decode_workspace_bytes_ex(B, Hq, Hkv, D, workers)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = A.load_library().attn_decode_paged_full(
        p(q), p(kc), p(vc), p(bt), p(ctx), p(o), p(lse), B, Hq, Hkv, D, 16, scale,
        int(bt.shape[1]), nb, workers, p(ws), need, stream)
    assert rc == 0, A.attn_last_error()
    return ws


@pytest.mark.parametrize("workers", [0, 300])
def test_noalloc_matches_ex_twice_second_smaller(workers):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    cases = [
        # the decode workload's shape, then a smaller batch with other context lengths
        dict(B=64, Hq=32, Hkv=8, D=128, block_size=16, ctx_lo=512, ctx_hi=4096, seed=1004),
        dict(B=5, Hq=8, Hkv=2, D=128, block_size=16, ctx_lo=0, ctx_hi=300, seed=77),
    ]
    for case in cases:
        print(f"noalloc decode case {case} workers={workers}", flush=True)
        d = W.decode_inputs(**case)
        q, kc, vc, bt, ctx = _upload(d, dev)
        scale = float(np.float32(1.0 / np.sqrt(case["D"])))
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        l1 = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        l2 = torch.empty_like(l1)
        _c_noalloc(q, kc, vc, bt, ctx, o1, l1, scale, workers)
        ws = _c_ex(q, kc, vc, bt, ctx, o2, l2, scale, workers)
        torch.cuda.synchronize()
        del ws
        assert torch.equal(o1, o2)
        assert torch.equal(l1, l2)
        O, L = oracle.decode_paged(d.q, d.k_cache, d.v_cache, d.block_table, d.ctx_lens, 16,
                                   scale=scale)
        mx, mn = check_bf16(to_np(o1), O)
        err = check_lse(to_np(l1), L)
        print(f"  O max {mx:.3e} mean {mn:.3e}; LSE max {err:.3e}", flush=True)


def test_noalloc_refuses_what_does_not_fit():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    cap = A.attn_decode_noalloc_max_bytes()
    d = W.decode_inputs(B=2, Hq=4, Hkv=1, D=64, block_size=16, ctx_lo=1, ctx_hi=40, seed=5)
    q, kc, vc, bt, ctx = _upload(d, dev)
    workers = 65536
    assert A.attn_decode_workspace_bytes_ex(2, 4, 1, 64, workers) > cap
    with pytest.raises(A.AttnError, match="fixed scratch"):
        A.attn_decode_paged_noalloc(q, kc, vc, bt, ctx, num_workers=workers)
