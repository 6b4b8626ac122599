#!/usr/bin/env python3
"""Benchmark of the fused exact-attention hot path on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  * prefill: attn_fwd on the 32K-token workload (B=1, Hq=32, Hkv=8, S=32768, D=128, bf16,
    causal, inputs N(0,1) x 0.5), the largest prefill configuration; then
  * decode:  attn_decode_paged on the paged workload (B=64, Hq=32, Hkv=8, D=128, contexts
    uniform in [512, 4096], 16-token blocks placed by a seeded permutation), which runs the
    split-KV stream kernel and the LSE-merge combine kernel.
Inputs are generated once, uploaded, and resident in HBM before timing starts. Between the two,
512 MiB of scratch memory is read (``--flush-mib``), so the decode starts with none of its K/V in
L2 or the memory-side cache; the flush is outside both kernels' timed intervals but inside the
step's wall time (``ms_per_step``).

Printed (one JSON line): ``value`` is the 32K prefill's throughput in TFLOP/s counting 4*D
flops per visible (query, key) pair (causal-adjusted), from the median kernel duration over the
timed steps (the minimum is reported too); ``decode`` gives the decode KV bandwidth in GB/s
counting each visible token's K and V once plus q, o and the block table. Kernel durations come
from HIP events recorded around each launch on the launch stream (created without the
system-scope fence, so recording them adds no cache flush between kernels). ``roofline``
compares the 32K prefill with the bf16 dense MFMA peak, ``decode.roofline`` the decode with the
HBM peak. ``prefill_configs`` times the other bf16 prefill workloads (B=8, H=32, S=4096 and the
Llama-3-8B-shaped S=2048) the same way. ``clock`` is the graphics clock sampled while the 32K
prefill runs, with the fraction of the peak at that clock. ``cpu_baseline`` times the fp64 CPU
oracle on one query head of the 32K workload.
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
PREFILL = W.CONFIGS["long_s32768"]
EXTRA_PREFILLS = ("batched_b8_s4096", "llama3_8b_prefill")
DECODE = W.CONFIGS["paged_decode_b64"]
NOMINAL_CLOCK_MHZ = 2400.0
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


def cpu_baseline(min_seconds: float, cfg, q, k, v):
    """The fp64 oracle (as it stands) on one query head of prefill workload cfg (q, k, v: that
    head and its KV head, [1, 1, S, D]), repeated until min_seconds have passed."""
    import oracle
    from threadpoolctl import threadpool_info
    one = W.FwdConfig("one_head", 1, 1, 1, cfg.Sq, cfg.Sk, cfg.D, cfg.dtype, cfg.causal,
                      cfg.seed)
    flops = prefill_flops(one)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(q, k, v, causal=cfg.causal, scale=cfg.scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"one of the {cfg.Hq} query heads of {cfg.name} (1 x {cfg.Sq} x {cfg.Sk}, "
                      f"{'causal' if cfg.causal else 'full'}, fp64 numpy, dense score rows in "
                      f"slabs) x {reps} in {el:.1f} s; host cpus "
                      f"{os.cpu_count()}, affinity {len(os.sched_getaffinity(0))}"}


class ClockSampler:
    """Samples the GPU's current graphics clock from the driver (amdsmi) on a host thread while
    a timed region runs. Returns None when the library or the metric is unavailable."""

    def __init__(self, period_s=0.005):
        self.period = period_s
        self.samples = []
        self._stop = False
        self._th = None
        self._h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:
            self._h = None

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        vals = m.get("current_gfxclks")
        if isinstance(vals, (list, tuple)):
            vals = [float(x) for x in vals if isinstance(x, (int, float)) and 0 < x < 10000]
            if vals:
                return sum(vals) / len(vals)
        v = m.get("current_gfxclk", m.get("average_gfxclk_frequency"))
        return float(v) if isinstance(v, (int, float)) and 0 < v < 10000 else None

    def start(self):
        import threading
        if self._h is None:
            return self

        def run():
            while not self._stop:
                try:
                    v = self._read()
                    if v is not None:
                        self.samples.append(v)
                except Exception:
                    return
                time.sleep(self.period)

        self._th = threading.Thread(target=run, daemon=True)
        self._th.start()
        return self

    def stop(self):
        self._stop = True
        if self._th is not None:
            self._th.join()
        if self._h is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:
                pass
        if not self.samples:
            return None
        return float(np.median(self.samples))


def time_prefill(A, torch, dev, cfg, stream, warmup, reps):
    """Median and minimum duration of attn_fwd on workload cfg, each launch between its own
    fence-free events, after warm-up launches."""
    q, k, v = W.fwd_inputs_for(cfg)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)
    qg, kg, vg = bf(q), bf(k), bf(v)
    del q, k, v
    o = torch.empty_like(qg)
    lse = torch.empty(qg.shape[:3], dtype=torch.float32, device=dev)
    call = lambda: A.attn_fwd(qg, kg, vg, causal=cfg.causal, scale=float(cfg.scale), out=o,
                              lse=lse)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = HipEvents(2 * reps)
    for i in range(reps):
        ev.record(2 * i, stream)
        call()
        ev.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    ms = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)])
    ev.close()
    flops = prefill_flops(cfg)
    med, mn = float(np.median(ms)), float(np.min(ms))
    tf = flops / (med * 1e-3) / 1e12
    return {"workload": f"{cfg.name}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} S={cfg.Sq} D={cfg.D} "
                        f"causal bf16",
            "flops_per_launch": flops, "reps": reps, "warmup": warmup,
            "kernel_ms_median": round(med, 5), "kernel_ms_min": round(mn, 5),
            "tflops": round(tf, 2), "tflops_at_min": round(flops / (mn * 1e-3) / 1e12, 2),
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


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


def floor_timing(torch, dev, flush, flush_sink, stream, reps):
    """The floor the small kernels sit on, timed exactly as they are (alone between fence-free
    events, after the read flush): a kernel that writes one element, and torch's device copies
    of 4 MiB (the size of the 64 x 8192 norm's traffic) and 48 MiB (the 2048-token RoPE chunk's)."""
    one = torch.zeros(1, device=dev)
    bufs = {}
    for mib in (4, 48):
        a = torch.zeros((mib << 20) // 4, device=dev)
        bufs[mib] = (a, torch.empty_like(a))
    cases = [("fill_1_element_us", lambda: one.fill_(1.0)),
             ("device_copy_4MiB_us", lambda: bufs[4][1].copy_(bufs[4][0])),
             ("device_copy_48MiB_us", lambda: bufs[48][1].copy_(bufs[48][0]))]
    out = {}
    for name, fn in cases:
        fn()
        torch.cuda.synchronize()
        ev = HipEvents(2 * reps)
        for i in range(reps):
            if flush is not None:
                torch.amax(flush, dim=0, out=flush_sink)
            ev.record(2 * i, stream)
            fn()
            ev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
        out[name] = round(float(np.median([ev.elapsed_ms(2 * i, 2 * i + 1)
                                           for i in range(reps)])) * 1e3, 2)
        ev.close()
    del bufs, one
    return out


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


def paged_prefill_flops(cfg) -> float:
    """4*D flops per visible (query, key) pair, summed over the sequences of the batch."""
    total = 0
    for n, ctx in zip(cfg.q_lens, cfg.ctx_lens):
        i = np.arange(n, dtype=np.int64)
        total += int(np.clip(i + (ctx - n) + 1, 0, ctx).sum()) if cfg.causal else n * ctx
    return 4.0 * cfg.Hq * cfg.D * total


def paged_prefill_timing(A, torch, dev, stream, reps):
    """Prefill through the paged cache (attn_fwd_paged): the 512-token chunk over a 4096-token
    context, and a mixed batch of eight sequences' chunks; timed back to back."""
    out = {}
    for name, cfg in W.PAGED_PREFILL_CONFIGS.items():
        x = W.paged_prefill_inputs_for(cfg)
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        q, kc, vc = bf(x.q), bf(x.k_cache), bf(x.v_cache)
        bt, cu, ctx = i32(x.block_table), i32(x.cu_seqlens_q), i32(x.ctx_lens)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
        max_q, max_ctx = max(cfg.q_lens), max(cfg.ctx_lens)
        call = lambda: A.attn_fwd_paged(q, kc, vc, bt, cu, ctx, max_q, max_ctx,
                                        causal=cfg.causal, scale=float(cfg.scale), out=o,
                                        lse=lse)
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
        flops = paged_prefill_flops(cfg)
        tf = flops / (us * 1e-6) / 1e12
        out[name] = {"workload": f"Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} chunks {list(cfg.q_lens)} "
                                 f"over contexts {list(cfg.ctx_lens)}, 16-token blocks, "
                                 f"{'causal (bottom-right)' if cfg.causal else 'no mask'} bf16",
                     "us": round(us, 2), "flops_per_launch": flops, "tflops": round(tf, 2),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "key_splits": A.attn_fwd_paged_workspace_bytes(
                         len(cfg.q_lens), int(sum(cfg.q_lens)), cfg.Hq, cfg.Hkv, cfg.D, max_q,
                         max_ctx, cfg.causal) > 0}
        del q, kc, vc, bt, cu, ctx, o, lse
    return out


class HipGraph:
    """Stream capture into a hipGraph and its launch, through the HIP runtime's own entry points
    (ctypes), so replays cost no framework code on the host."""

    def __init__(self):
        import ctypes
        import exact_attention_42_amd as A
        rts = A._hip_runtimes_mapped()
        if len(rts) != 1:
            raise RuntimeError(f"expected one HIP runtime in the process, found {rts}")
        self.ct = ctypes
        h = ctypes.CDLL(rts[0])
        vp = ctypes.c_void_p
        h.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
        h.hipStreamEndCapture.argtypes = [vp, ctypes.POINTER(vp)]
        h.hipGraphInstantiate.argtypes = [ctypes.POINTER(vp), vp, vp, ctypes.c_char_p,
                                          ctypes.c_size_t]
        h.hipGraphLaunch.argtypes = [vp, vp]
        h.hipGraphExecDestroy.argtypes = [vp]
        h.hipGraphDestroy.argtypes = [vp]
        self.h = h
        self.graph = vp()
        self.exec = vp()

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")

    def capture(self, stream, fn):
        ct = self.ct
        self._ok(self.h.hipStreamBeginCapture(ct.c_void_p(stream), 0), "hipStreamBeginCapture")
        try:
            fn()
        finally:
            self._ok(self.h.hipStreamEndCapture(ct.c_void_p(stream), ct.byref(self.graph)),
                     "hipStreamEndCapture")
        self._ok(self.h.hipGraphInstantiate(ct.byref(self.exec), self.graph, None, None, 0),
                 "hipGraphInstantiate")

    def launch(self, stream):
        self._ok(self.h.hipGraphLaunch(self.exec, self.ct.c_void_p(stream)), "hipGraphLaunch")

    def close(self):
        if self.exec:
            self.h.hipGraphExecDestroy(self.exec)
        if self.graph:
            self.h.hipGraphDestroy(self.graph)


def decode_graph_timing(A, torch, dq, dkc, dvc, dbt, dctx, scale, reps):
    """A whole decode step -- RoPE + paged cache store of the 64 new tokens, then the paged
    decode (stream + combine kernels) -- captured once into a hipGraph (caller workspace) and
    launched with hipGraphLaunch, against the same step enqueued eagerly through the binding:
    GPU time per step (events around all steps, back to back) and host time per enqueue."""
    dev = dq.device
    B, Hq, D = dq.shape
    Hkv = dkc.shape[1]
    rng = np.random.default_rng(17)
    mk = lambda shape: torch.from_numpy(
        W.bf16_round(rng.standard_normal(shape, dtype=np.float32))).to(dev).to(torch.bfloat16)
    rq, rk, rv = mk((B, Hq, D)), mk((B, Hkv, D)), mk((B, Hkv, D))
    pos = (dctx - 1).to(torch.int32)
    qrot = torch.empty_like(rq)
    kc, vc = dkc.clone(), dvc.clone()
    ws = torch.empty(A.attn_decode_workspace_bytes_ex(B, Hq, Hkv, D, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty_like(dq)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    sptr = side.cuda_stream

    def step():
        A.rope_cache_write(rq, rk, rv, pos, kc, vc, dbt, q_out=qrot, stream=side)
        A.attn_decode_paged_full(qrot, kc, vc, dbt, dctx, scale=scale, out=out, lse=lse,
                               workspace=ws, stream=side)

    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    g = HipGraph()
    g.capture(sptr, step)
    torch.cuda.synchronize()
    ev = HipEvents(4)
    res = {}
    for k_, (name, fn) in enumerate((("eager", step), ("graph", lambda: g.launch(sptr)))):
        fn()
        torch.cuda.synchronize()
        ev.record(2 * k_, sptr)
        h0 = time.perf_counter()
        for _ in range(reps):
            fn()
        h1 = time.perf_counter()
        ev.record(2 * k_ + 1, sptr)
        torch.cuda.synchronize()
        res[name] = (ev.elapsed_ms(2 * k_, 2 * k_ + 1) * 1e3 / reps, (h1 - h0) * 1e6 / reps)
    ev.close()
    g.close()
    return {"step": "rope_cache_write (64 tokens) + attn_decode_paged_ex", "steps": reps,
            "gpu_us_per_step_eager": round(res["eager"][0], 2),
            "gpu_us_per_step_graph": round(res["graph"][0], 2),
            "host_us_per_enqueue_eager": round(res["eager"][1], 2),
            "host_us_per_enqueue_graph": round(res["graph"][1], 2),
            "note": "hipGraphLaunch through ctypes; back to back, no cache flush in between"}


def progress(msg):
    """A progress line on stderr (the JSON result is the only line on stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time for the oracle baseline (0 skips it)")
    ap.add_argument("--extra-reps", type=int, default=50,
                    help="timed launches of each other bf16 prefill workload (0 = skip them)")
    ap.add_argument("--norm-reps", type=int, default=20,
                    help="timed launches of the fused add_rms_norm, of the RoPE + cache write "
                         "and of the chunked prefill per shape (0 = skip all three)")
    ap.add_argument("--graph-reps", type=int, default=50,
                    help="decode steps launched as a hipGraph and eagerly (0 = skip that part)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="scratch MiB read before each decode, outside its timing "
                         "(0 = none)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for counter scaling)")
    ap.add_argument("--prefill", default=PREFILL.name, choices=[
                        n for n, c in W.CONFIGS.items() if c.kind == "fwd" and c.dtype == "bf16"],
                    help="prefill workload of the step (default: the 32K-token one; the others "
                         "are for profiling runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)
    pcfg = W.CONFIGS[args.prefill]

    import torch
    import exact_attention_42_amd as A

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch.bfloat16)

    q, k, v = W.fwd_inputs_for(pcfg)
    qg, kg, vg = bf(q), bf(k), bf(v)
    head0 = (q[:, :1].copy(), k[:, :1].copy(), v[:, :1].copy())   # for the CPU baseline
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
    scale_p, scale_d = float(pcfg.scale), float(DECODE.scale)

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
        A.attn_fwd(qg, kg, vg, causal=pcfg.causal, scale=scale_p, out=o, lse=lse)
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

    progress(f"inputs resident ({pcfg.name} + {DECODE.name}); {args.warmup} warm-up steps")
    for _ in range(args.warmup):
        step()
    ev = HipEvents(4 * args.steps)
    torch.cuda.synchronize()
    clock = ClockSampler().start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clock_mhz = clock.stop()

    fwd = np.array([ev.elapsed_ms(4 * i, 4 * i + 1) for i in range(args.steps)])
    dec = np.array([ev.elapsed_ms(4 * i + 2, 4 * i + 3) for i in range(args.steps)])
    ev.close()
    fwd_ms, fwd_min = float(np.median(fwd)), float(np.min(fwd))
    dec_ms, dec_min = float(np.median(dec)), float(np.min(dec))
    del qg, kg, vg, o, lse
    torch.cuda.empty_cache()
    progress(f"{args.steps} steps timed: prefill median {fwd_ms:.4f} ms, decode median "
             f"{dec_ms:.4f} ms")
    extras = {}
    if args.extra_reps > 0:
        for name in EXTRA_PREFILLS:
            if name != pcfg.name:
                progress(f"timing {name}")
                extras[name] = time_prefill(A, torch, dev, W.CONFIGS[name], stream,
                                            min(10, args.extra_reps), args.extra_reps)
                torch.cuda.empty_cache()
    graph = decode_graph_timing(A, torch, dq, dkc, dvc, dbt, dctx, scale_d, args.graph_reps) \
        if args.graph_reps > 0 else None
    norm = norm_timing(A, torch, dev, flush, flush_sink, stream, args.norm_reps) \
        if args.norm_reps > 0 else None
    rope = rope_timing(A, torch, dev, dq, dkc, dvc, dbt, dctx, flush, flush_sink, stream,
                       args.norm_reps) if args.norm_reps > 0 else None
    floor = floor_timing(torch, dev, flush, flush_sink, stream, args.norm_reps) \
        if args.norm_reps > 0 else None
    chunk = chunked_prefill_timing(A, torch, dev, stream, 20) if args.norm_reps > 0 else None
    paged = paged_prefill_timing(A, torch, dev, stream, 20) if args.norm_reps > 0 else None
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    flops = prefill_flops(pcfg)
    tflops = flops / (fwd_ms * 1e-3) / 1e12
    dbytes = decode_bytes(ctx_lens, DECODE)
    gbs = dbytes / (dec_ms * 1e-3) / 1e9

    fwd_digest = source_digest("attn_fwd_bf16.hip", "attn_fwd_wide.hip", "fwd_tiles.hpp",
                               "cdna4.hpp")
    dec_digest = source_digest("attn_decode.hip", "cdna4.hpp", "attn_api.hip")
    clock_info = None
    if clock_mhz is not None:
        clock_info = {"gfx_mhz_median_during_prefill": round(clock_mhz, 1),
                      "nominal_mhz": NOMINAL_CLOCK_MHZ,
                      "peak_at_that_clock_tflops": round(
                          PEAK_BF16_TFLOPS * clock_mhz / NOMINAL_CLOCK_MHZ, 1),
                      "frac_of_peak_at_that_clock": round(
                          tflops / (PEAK_BF16_TFLOPS * clock_mhz / NOMINAL_CLOCK_MHZ), 4)}
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
        "data": f"synthetic (seeded N(0,1) inputs rounded to bf16; seeds {pcfg.seed} and "
                f"{DECODE.seed})",
        "config": {
            "workload": f"{pcfg.name}: B={pcfg.B} Hq={pcfg.Hq} Hkv={pcfg.Hkv} S={pcfg.Sq} "
                        f"D={pcfg.D} causal bf16"
                        + (f" (inputs x{pcfg.input_scale})" if pcfg.input_scale != 1.0 else "")
                        + " + paged_decode_b64: B=64 Hq=32 Hkv=8 D=128 ctx U[512,4096] block 16",
            "prefill_flops_per_launch": flops,
            "decode_bytes_per_launch": dbytes,
            "sum_ctx": int(np.sum(ctx_lens)),
            "cache_flush_mib_before_decode": args.flush_mib,
        },
        "prefill": {"kernel_ms_median": round(fwd_ms, 5), "kernel_ms_min": round(fwd_min, 5),
                    "tflops": round(tflops, 2),
                    "tflops_at_min": round(flops / (fwd_min * 1e-3) / 1e12, 2),
                    "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)},
        "decode": {"kernel_ms_median": round(dec_ms, 5), "kernel_ms_min": round(dec_min, 5),
                   "value": round(gbs, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": measured_traffic("decode_stream_paged_decode_b64",
                                                            dec_digest)}},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(f"fwd_bf16_{pcfg.name}", fwd_digest)},
        "clock": clock_info,
        "prefill_configs": extras,
        "kernel_source_digest": {"fwd": fwd_digest, "decode": dec_digest},
    }
    if graph is not None:
        out["decode"]["hipgraph"] = graph
    if norm is not None:
        out["add_rms_norm"] = norm
    if rope is not None:
        out["rope_cache_write"] = rope
    if floor is not None:
        out["small_kernel_floor"] = floor
    if chunk is not None:
        out["chunked_prefill"] = chunk
    if paged is not None:
        out["paged_prefill"] = paged
    if args.cpu_seconds > 0:
        progress("timing the fp64 oracle on the host")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds, pcfg, *head0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
