#!/usr/bin/env python3
"""Benchmark of the fused exact-attention hot path on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  * prefill: attn_fwd on the Llama-3-8B-shaped workload (B=1, Hq=32, Hkv=8, S=2048, D=128,
    bf16, causal), then
  * decode:  attn_decode_paged on the paged workload (B=64, Hq=32, Hkv=8, D=128, contexts
    uniform in [512, 4096], 16-token blocks placed by a seeded permutation), which runs the
    split-KV stream kernel and the LSE-merge combine kernel.
Inputs are generated once, uploaded, and resident in HBM before timing starts. Between the two,
512 MiB of scratch memory is read (``--flush-mib``), so the decode starts with none of its K/V in
L2 or the memory-side cache; the flush is outside both kernels' timed intervals but inside the
step's wall time (``ms_per_step``).

Printed (one JSON line): ``value`` is the prefill kernel's throughput in TFLOP/s counting
4*D flops per visible (query, key) pair (causal-adjusted); ``decode`` gives the decode KV
bandwidth in GB/s counting each visible token's K and V once plus q, o and the block table.
Kernel durations come from HIP events recorded around each launch on the launch stream
(created without the system-scope fence, so recording them adds no cache flush between kernels).
``roofline`` compares the prefill kernel with the bf16 dense MFMA peak, ``decode.roofline``
the decode with the HBM peak. ``cpu_baseline`` times the fp64 CPU oracle on the host on the
same prefill workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CUs x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PREFILL = W.CONFIGS["llama3_8b_prefill"]
DECODE = W.CONFIGS["paged_decode_b64"]
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_attention_42_amd", "csrc")


def prefill_flops(cfg) -> float:
    """4*D flops per visible (query, key) pair: QK^T and PV each 2*D per pair."""
    Sq, Sk = cfg.Sq, cfg.Sk
    if cfg.causal:
        i = np.arange(Sq, dtype=np.int64)
        visible = int(np.clip(i + (Sk - Sq) + 1, 0, Sk).sum())
    else:
        visible = Sq * Sk
    return 4.0 * cfg.B * cfg.Hq * cfg.D * visible


def decode_bytes(ctx_lens, cfg) -> float:
    """Each visible token's K and V once per KV head, plus q, o and the block table rows."""
    kv = float(np.sum(ctx_lens, dtype=np.int64)) * 2 * cfg.Hkv * cfg.D * 2
    qo = 2 * cfg.B * cfg.Hq * cfg.D * 2
    nblk = (np.asarray(ctx_lens, dtype=np.int64) + cfg.block_size - 1) // cfg.block_size
    table = float(nblk.sum()) * 4 + cfg.B * 4
    return kv + qo + table


def source_digest(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_tag: str, digest: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on the current
    kernel source (its digest line matches); otherwise None."""
    path = os.path.join(PROFILES, f"{kernel_tag}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_d = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    m_t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_d or not m_t or m_d.group(1) != digest:
        return None
    return float(m_t.group(1))


class HipEvents:
    """Timing events from the HIP runtime torch already loaded, created with
    hipEventDisableSystemFence: recording one then costs no system-scope cache writeback and
    invalidation, which with ordinary events adds a bubble of several microseconds in front
    of the next kernel and slows it (the HIP header documents the flag for exactly this)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        import torch  # noqa: F401  (maps the runtime)
        import exact_attention_42_amd as A
        rts = A._hip_runtimes_mapped()
        if len(rts) != 1:
            raise RuntimeError(f"expected one HIP runtime in the process, found {rts}")
        self._ct = ctypes
        self._hip = ctypes.CDLL(rts[0])
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self._hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.ev.append(e)

    def record(self, i, stream):
        rc = self._hip.hipEventRecord(self.ev[i], self._ct.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, i, j):
        t = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(t), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(t.value)

    def close(self):
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


def cpu_baseline(min_seconds: float):
    """The fp64 oracle (as it stands) on the prefill workload, repeated until min_seconds."""
    import oracle
    from threadpoolctl import threadpool_info
    q, k, v = W.fwd_inputs_for(PREFILL)
    flops = prefill_flops(PREFILL)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(q, k, v, causal=PREFILL.causal, scale=PREFILL.scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"full llama3_8b_prefill workload (32 heads x 2048 x 2048, causal, fp64 "
                      f"numpy, dense score rows) x {reps} in {el:.1f} s; host cpus "
                      f"{os.cpu_count()}, affinity {len(os.sched_getaffinity(0))}"}


def norm_timing(A, torch, dev, flush, flush_sink, stream, reps):
    """The fused residual-add RMS norm on the page's (64, 8192) bf16 tensor and on an
    8192-wide hidden state over 16384 tokens. Each launch is timed alone with fence-free
    events, after the same 512 MiB read flush as the decode. Algorithmic bytes: x and the
    residual read, out and the new residual written (8 B per element) plus the weight row."""
    res = {}
    for name in ("add_rms_norm_64x8192", "add_rms_norm_16384x8192"):
        cfg = W.NORM_CONFIGS[name]
        x, r, w = W.norm_inputs_for(cfg)
        gx = torch.from_numpy(x).to(dev).to(torch.bfloat16)
        gr = torch.from_numpy(r).to(dev).to(torch.bfloat16)
        gw = torch.from_numpy(w).to(dev).to(torch.bfloat16)
        del x, r, w
        out, tres = torch.empty_like(gx), torch.empty_like(gx)
        A.add_rms_norm(gx, gr, gw, eps=cfg.eps, out=out, residual_out=tres)
        torch.cuda.synchronize()
        ev = HipEvents(2 * reps)
        for i in range(reps):
            if flush is not None:
                torch.amax(flush, dim=0, out=flush_sink)
            ev.record(2 * i, stream)
            A.add_rms_norm(gx, gr, gw, eps=cfg.eps, out=out, residual_out=tres)
            ev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
        us = float(np.median([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)])) * 1e3
        ev.close()
        nbytes = 8.0 * cfg.M * cfg.d + 2.0 * cfg.d
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "bytes_per_launch": nbytes, "GB/s": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        del gx, gr, gw, out, tres
    return res


def rope_timing(A, torch, dev, dq, dkc, dvc, dbt, dctx, flush, flush_sink, stream, reps):
    """The fused RoPE + paged cache store: (1) the decode step's 64 new tokens (one per
    sequence, at position ctx - 1, into the decode workload's own cache: the step that
    precedes the decode), (2) a 2048-token prefill chunk of one sequence into a 128-block
    pool. Each launch timed alone after the read flush. Algorithmic bytes: q, k, v read,
    rotated q written, k and v stored (2 B per element each way) plus positions and table."""
    B, Hq, D = dq.shape
    Hkv = dkc.shape[1]
    res = {}
    rng = np.random.default_rng(7)
    cases = []
    pos = (dctx - 1).to(torch.int32)
    mk = lambda shape: torch.from_numpy(
        W.bf16_round(rng.standard_normal(shape, dtype=np.float32))).to(dev).to(torch.bfloat16)
    cases.append(("decode_step_b64", mk((B, Hq, D)), mk((B, Hkv, D)), mk((B, Hkv, D)), pos,
                  dkc, dvc, dbt, None))
    T, nb = 2048, 128
    cases.append(("prefill_chunk_2048", mk((T, Hq, D)), mk((T, Hkv, D)), mk((T, Hkv, D)),
                  torch.arange(T, dtype=torch.int32, device=dev),
                  torch.zeros((nb, Hkv, 16, D), dtype=torch.bfloat16, device=dev),
                  torch.zeros((nb, Hkv, 16, D), dtype=torch.bfloat16, device=dev),
                  torch.from_numpy(rng.permutation(nb).astype(np.int32)[None, :]).to(dev),
                  torch.zeros(T, dtype=torch.int32, device=dev)))
    for name, q, k, v, p, kc, vc, bt, seq in cases:
        qo = torch.empty_like(q)
        A.rope_cache_write(q, k, v, p, kc, vc, bt, seq_ids=seq, q_out=qo)
        torch.cuda.synchronize()
        ev = HipEvents(2 * reps)
        for i in range(reps):
            if flush is not None:
                torch.amax(flush, dim=0, out=flush_sink)
            ev.record(2 * i, stream)
            A.rope_cache_write(q, k, v, p, kc, vc, bt, seq_ids=seq, q_out=qo)
            ev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
        us = float(np.median([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)])) * 1e3
        ev.close()
        t = q.shape[0]
        nbytes = 2.0 * t * D * (2 * Hq + 4 * Hkv) + 8.0 * t
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"tokens": t, "us": round(us, 2), "bytes_per_launch": nbytes,
                     "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return res


def chunked_prefill_timing(A, torch, dev, stream, reps):
    """The chunked-prefill step (§8(f) N3 workload): the last 512 tokens of a 4096-token
    prompt against the whole prefix, bottom-right causal. Its 128 query tiles cannot fill the
    device, so the forward splits each tile's keys; timed back to back (compute-bound)."""
    cfg = W.CONFIGS["chunked_prefill_512_of_4096"]
    q, k, v = W.fwd_inputs_for(cfg)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)
    qg, kg, vg = bf(q), bf(k), bf(v)
    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device=dev)
    call = lambda: A.attn_fwd(qg, kg, vg, causal=True, scale=float(cfg.scale), out=o, lse=lse)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = HipEvents(2)
    ev.record(0, stream)
    for _ in range(reps):
        call()
    ev.record(1, stream)
    torch.cuda.synchronize()
    us = ev.elapsed_ms(0, 1) * 1e3 / reps
    ev.close()
    tf = prefill_flops(cfg) / (us * 1e-6) / 1e12
    return {"workload": "B=1 Hq=32 Hkv=8 Sq=512 Sk=4096 D=128 causal (bottom-right) bf16",
            "us": round(us, 2), "flops_per_launch": prefill_flops(cfg),
            "tflops": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "key_splits": A.attn_fwd_workspace_bytes(1, 32, 8, 512, 4096, 128, True) > 0}


def decode_graph_timing(A, torch, dq, dkc, dvc, dbt, dctx, scale, stream, reps):
    """The decode (stream + combine kernels) captured once into a hipGraph through
    attn_decode_paged_ex with a caller workspace, then replayed back to back: GPU time per
    replay (events around all replays) and host time per enqueue, against the same number of
    eager calls through the Python binding."""
    B, Hq, D = dq.shape
    Hkv = dkc.shape[1]
    ws = torch.empty(A.attn_decode_workspace_bytes(B, Hq, Hkv, D, 0), dtype=torch.uint8,
                     device=dq.device)
    out = torch.empty_like(dq)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dq.device)

    def call():
        A.attn_decode_paged_ex(dq, dkc, dvc, dbt, dctx, scale=scale, out=out, lse=lse,
                               workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    ev = HipEvents(4)
    res = {}
    for name, fn in (("eager", call), ("graph", g.replay)):
        fn()
        torch.cuda.synchronize()
        ev.record(2 * (name == "graph"), stream)
        h0 = time.perf_counter()
        for _ in range(reps):
            fn()
        h1 = time.perf_counter()
        ev.record(2 * (name == "graph") + 1, stream)
        torch.cuda.synchronize()
        res[name] = (ev.elapsed_ms(2 * (name == "graph"), 2 * (name == "graph") + 1) * 1e3 / reps,
                     (h1 - h0) * 1e6 / reps)
    ev.close()
    return {"replays": reps,
            "gpu_us_per_call_eager": round(res["eager"][0], 2),
            "gpu_us_per_call_graph": round(res["graph"][0], 2),
            "host_us_per_enqueue_eager": round(res["eager"][1], 2),
            "host_us_per_enqueue_graph": round(res["graph"][1], 2),
            "note": "back to back, no cache flush in between"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time for the oracle baseline (0 skips it)")
    ap.add_argument("--norm-reps", type=int, default=20,
                    help="timed launches of the fused add_rms_norm and of the RoPE + cache "
                         "write per shape (0 = skip both)")
    ap.add_argument("--graph-reps", type=int, default=50,
                    help="replays of the decode captured in a hipGraph (0 = skip that part)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="scratch MiB read before each decode, outside its timing "
                         "(0 = none)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_42_amd as A

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)

    q, k, v = W.fwd_inputs_for(PREFILL)
    qg, kg, vg = bf(q), bf(k), bf(v)
    del q, k, v
    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device=dev)
    d = W.decode_inputs_for(DECODE)
    dq, dkc, dvc = bf(d.q), bf(d.k_cache), bf(d.v_cache)
    dbt = torch.from_numpy(d.block_table).to(dev)
    dctx = torch.from_numpy(d.ctx_lens).to(dev)
    do = torch.empty_like(dq)
    ctx_lens = d.ctx_lens.copy()
    del d
    scale_p, scale_d = float(PREFILL.scale), float(DECODE.scale)

    stream = torch.cuda.current_stream().cuda_stream

    # Read once before every decode, outside its timed interval: 512 MiB is twice the MI355X's
    # 256 MiB memory-side cache, so the decode finds none of its 624 MB of K/V left in a cache
    # by the previous step (a serving loop runs other layers in between). A read, not a write:
    # written scratch would leave dirty lines whose write-back then lands inside the decode.
    flush = torch.zeros((args.flush_mib << 20) // 4, dtype=torch.int32, device=dev) \
        if args.flush_mib > 0 else None
    flush_sink = torch.zeros((), dtype=torch.int32, device=dev)

    def step(i=None):
        # events e0 | prefill | e1 | cache flush | e2 | decode (stream + combine) | e3, all on
        # the launch stream
        if i is not None:
            ev.record(4 * i, stream)
        A.attn_fwd(qg, kg, vg, causal=True, scale=scale_p, out=o, lse=lse)
        if i is not None:
            ev.record(4 * i + 1, stream)
        if flush is not None:
            torch.amax(flush, dim=0, out=flush_sink)
        if i is not None:
            ev.record(4 * i + 2, stream)
        A.attn_decode_paged(dq, dkc, dvc, dbt, dctx, scale=scale_d, out=do)
        if i is not None:
            ev.record(4 * i + 3, stream)

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    ev = HipEvents(4 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    fwd_ms = float(np.mean([ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(args.steps)]))
    dec_ms = float(np.mean([ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)]))
    ev.close()
    graph = decode_graph_timing(A, torch, dq, dkc, dvc, dbt, dctx, scale_d, stream,
                                args.graph_reps) if args.graph_reps > 0 else None
    norm = norm_timing(A, torch, dev, flush, flush_sink, stream, args.norm_reps) \
        if args.norm_reps > 0 else None
    rope = rope_timing(A, torch, dev, dq, dkc, dvc, dbt, dctx, flush, flush_sink, stream,
                       args.norm_reps) if args.norm_reps > 0 else None
    chunk = chunked_prefill_timing(A, torch, dev, stream, 20) if args.norm_reps > 0 else None
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    flops = prefill_flops(PREFILL)
    tflops = flops / (fwd_ms * 1e-3) / 1e12
    dbytes = decode_bytes(ctx_lens, DECODE)
    gbs = dbytes / (dec_ms * 1e-3) / 1e9

    fwd_digest = source_digest("attn_fwd_bf16.hip", "cdna4.hpp")
    dec_digest = source_digest("attn_decode.hip", "cdna4.hpp", "attn_api.hip")
    out = {
        "metric": "fwd attention TFLOP/s & % MFMA peak (prefill); decode KV GB/s & % HBM peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs rounded to bf16; seeds 1002 and 1004)",
        "config": {
            "workload": "llama3_8b_prefill: B=1 Hq=32 Hkv=8 S=2048 D=128 causal bf16 "
                        "+ paged_decode_b64: B=64 Hq=32 Hkv=8 D=128 ctx U[512,4096] "
                        "block 16",
            "prefill_flops_per_launch": flops,
            "decode_bytes_per_launch": dbytes,
            "sum_ctx": int(np.sum(ctx_lens)),
            "cache_flush_mib_before_decode": args.flush_mib,
        },
        "prefill": {"kernel_ms": round(fwd_ms, 5), "tflops": round(tflops, 2),
                    "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)},
        "decode": {"kernel_ms": round(dec_ms, 5), "value": round(gbs, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": measured_traffic("decode_stream_paged_decode_b64",
                                                            dec_digest)}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("fwd_bf16_llama3_8b_prefill", fwd_digest)},
        "kernel_source_digest": {"fwd": fwd_digest, "decode": dec_digest},
    }
    if graph is not None:
        out["decode"]["hipgraph"] = graph
    if norm is not None:
        out["add_rms_norm"] = norm
    if rope is not None:
        out["rope_cache_write"] = rope
    if chunk is not None:
        out["chunked_prefill"] = chunk
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
