"""Benchmark of the attention core on one MI355X (synthetic, seeded inputs).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]
                    [--only CALL [--model flash|pro]]

Prints ONE JSON line.  The headline `value` is the windowed (SWA) prefill
throughput in algorithmic TFLOP/s on the 4 x 8192-token workload (64 q / 8 KV
heads, window 128, per-head sinks): in-window (q, k) pairs x 2 x (192 + 128)
flop, divided by the mean duration of one hsw_swa_prefill call (band kernel +
ring commit) measured with HIP events on the stream the kernels run on.
The same line carries the windowed-decode HBM GB/s on 256 sequences (the
second half of the metric), the other calls of the path, a roofline object
for the dominant kernel and the fp64 CPU oracle timed on a bounded sample.
Unless --quick, a `pro` object repeats every call and the hybrid step at
MiMo-V2.6-Pro shapes (128 q heads, 8 KV heads on both layer kinds, value
scale 0.612, 70 layers of which 10 full).

Inputs are resident in HBM before each timed region.  Timed regions cycle
over enough replicas of the inputs that every launch reads HBM rather than
the 256 MB Infinity Cache.  Every call is timed as 5 runs of N back-to-back
launches between two HIP events (N >= 200 for the windowed calls, >= 20 for
the full decode, >= 3 hybrid steps) and reported as the median run; the
runs themselves are kept for the headline call.  The GPU's clocks and power
(rocm-smi; clocks are not locked) and the host CPU model are recorded, and
the fp64 oracle is timed on workloads 1-4 in full and on a sample of the
hybrid step, extrapolated by row count and labelled so.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SWA decode HBM GB/s (% peak) + SWA prefill TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DEV = "cuda:0"
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hybrid_sliding_window_amd", "csrc")

# HBM bytes per call read by the TCC counters (FETCH_SIZE / WRITE_SIZE, scaled
# by a plain copy of known size) for the kernel sources whose digest is given;
# profiles/swa_prefill_4x8192_hbm_traffic.md,
# profiles/swa_decode_256seq_hbm_traffic.md and
# profiles/vit_window_16x4096_hbm_traffic.md hold the runs.  Reported as null
# once those sources differ from the ones measured.
MEASURED_TRAFFIC = {
    # sweep kernel 1014.0 MB read / 537.0 MB written + ring commit 2.7 / 2.6 MB
    "swa_prefill": (1556.3e6, ("swa_prefill.hip", "generic_attn.hip", "hsw_device.h"), "c99718e8e8ec1ca9"),
    "swa_decode": (178.46e6, ("swa_decode.hip", "hsw_device.h"), "896eeabc5cd54b5f"),
    # ViT window block: 202.4 MB read, 134.2 MB written
    "vit_window": (336.6e6, ("vit.hip", "hsw_device.h"), "5d83105600c1bde9"),
}


def measured_traffic(call):
    """Counter-measured HBM bytes per call, or None if the kernel changed."""
    import hashlib
    nbytes, files, digest = MEASURED_TRAFFIC[call]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return nbytes if h.hexdigest()[:16] == digest else None


def warm(fn, stream, seconds=0.3):
    """Call fn until `seconds` of wall time have passed, so the GPU clocks have
    ramped before anything is timed."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 16 == 0:
            stream.synchronize()
    stream.synchronize()


RUNS = 5   # timed runs per call; the median is reported


def ev_time(fn, n, stream, runs=None, reps=None):
    """Median over RUNS (or `reps`) runs of the mean ms per call of fn() over
    n back-to-back calls, each run bracketed by HIP events on `stream`.  The
    per-run means are appended to `runs` when given."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    per = []
    k = 0
    for r in range(reps or RUNS):
        start.record(stream)
        for i in range(n):
            fn(k)
            k += 1
        end.record(stream)
        end.synchronize()
        per.append(start.elapsed_time(end) / n)
    if runs is not None:
        runs.extend(per)
    return statistics.median(per)


def gpu_clocks_power():
    """The GPU's current clocks and power as rocm-smi reports them (a child
    process; clocks are not locked), or the error that prevented it."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True, text=True,
                           timeout=60)
        d = json.loads(r.stdout)
    except Exception as e:  # noqa: BLE001 - recorded, never fatal
        return {"error": f"rocm-smi: {type(e).__name__}: {str(e)[:160]}"}
    out = {}
    for card, vals in d.items():
        if isinstance(vals, dict):
            out[card] = {k: v for k, v in vals.items() if "clock" in k.lower() or "power" in k.lower()
                         or k.lower().startswith(("sclk", "mclk", "fclk", "socclk"))}
    if not any("power" in k.lower() for v in out.values() for k in v):
        # rocm-smi printed no power: the driver's hwmon average power, if readable
        import glob
        for f in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_average")
                        + glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")):
            try:
                with open(f) as fh:
                    out.setdefault("hwmon", {})[f.split("/device/")[0].rsplit("/", 1)[1] + " " +
                                             os.path.basename(f)] = f"{int(fh.read()) / 1e6:.1f} W"
            except (OSError, ValueError):
                pass
        if "hwmon" not in out:
            out["power"] = "not reported by rocm-smi or hwmon on this machine"
    return out


def host_cpu():
    """CPU model name (/proc/cpuinfo) and the cores this process sees."""
    name = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": name, "nproc": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def swa_prefill_pairs(lens, starts, window=128):
    """In-window (query, key) pairs per head: sum over rows of min(p + 1, W)."""
    tot = 0
    for n, s in zip(lens, starts):
        p = np.arange(s, s + n, dtype=np.int64)
        tot += int(np.minimum(p + 1, window).sum())
    return tot


def heads(model):
    return f"{model.n_q_heads} q / {model.swa_kv_heads} KV heads"


def bench_swa_prefill(hsw, wl, steps, warmup, stream, model=None):
    """Windowed prefill, 4 x 8192 tokens from position 0; also times the RoPE +
    staging write that feeds it."""
    model = model or wl.FLASH
    hq, hkv = model.n_q_heads, model.swa_kv_heads
    S, T1 = 4, 8192
    b = wl.swa_prefill_batch(seed=2, device=DEV, **wl.model_kw(model, "swa"))
    sh = b["shape"]
    T = S * T1
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in b.items()}
    q_rot = torch.empty_like(d["q"])
    kst = torch.empty_like(d["k"])
    vst = torch.empty_like(d["v"])

    def rope(i):
        hsw.hsw_rope_partial_kv_write(sh, T, d["q"], d["k"], d["v"], d["pos"], None, hsw.HSW_DST_STAGING,
                                      kst, vst, T, None, q_rot, None, stream)
    rope(0)
    out = torch.empty((T, hq, 128), dtype=torch.bfloat16, device=DEV)

    def call(i):
        hsw.hsw_swa_prefill(sh, S, T1, d["cu_seqlens"], d["start_pos"], q_rot, kst, vst, d["kring"],
                            d["vring"], d["sinks"], out, stream)
    for i in range(warmup):
        call(i)
        rope(i)
    warm(call, stream)
    runs = []
    n = max(steps, 200)
    t_call = ev_time(call, n, stream, runs)
    t_rope = ev_time(rope, n, stream)

    # the fused chain: K-only RoPE into staging, then the prefill that
    # rotates q itself (no q_rot written or read) and reads V in place (v's
    # layout is the staging one, so no V copy is written or read)
    def rope_kv(i):
        hsw.hsw_rope_partial_kv_write(sh, T, None, d["k"], None, d["pos"], None, hsw.HSW_DST_STAGING,
                                      kst, None, T, None, None, None, stream)

    def fused(i):
        hsw.hsw_swa_prefill_qrope(sh, S, T1, d["cu_seqlens"], d["start_pos"], d["q"], kst, d["v"], d["kring"],
                                  d["vring"], d["sinks"], out, stream)
    fused(0)
    warm(fused, stream)
    t_fused = ev_time(fused, n, stream)
    t_rope_kv = ev_time(rope_kv, n, stream)
    pairs = swa_prefill_pairs([T1] * S, [0] * S)
    flops = pairs * hq * 2 * (192 + 128)
    # algorithmic bytes: q_rot, staged K/V read once, out written once, the
    # ring commit (last 128 rows of K and V per sequence) written once
    bytes_ = T * hq * 192 * 2 + T * hkv * (192 + 128) * 2 + T * hq * 128 * 2 + S * hkv * 128 * (192 + 128) * 2
    rope_bytes = T * 2 * (hq * 192 + hkv * 192 + hkv * 128) * 2
    rope_kv_bytes = T * 2 * hkv * 192 * 2
    fused_res = dict(ms=t_fused, gbs=bytes_ / t_fused / 1e6, tflops=flops / t_fused / 1e9,
                     rope_kv_ms=t_rope_kv, rope_kv_gbs=rope_kv_bytes / t_rope_kv / 1e6,
                     chain_ms=t_rope_kv + t_fused, unfused_chain_ms=t_rope + t_call,
                     chain_bytes=rope_kv_bytes + bytes_, unfused_chain_bytes=rope_bytes + bytes_,
                     workload="K-only RoPE into staging + hsw_swa_prefill_qrope (q rotated in the kernel, V "
                              "read in place) against RoPE + hsw_swa_prefill, same workload")
    return dict(
        fused=fused_res,
        ms=t_call, runs_ms=runs, launches_per_run=n, flops=flops, bytes=bytes_, tokens=T,
        tflops=flops / t_call / 1e9, gbs=bytes_ / t_call / 1e6,
        frac_mfma_peak=flops / t_call / 1e9 / BF16_PEAK_TFLOPS, frac_hbm_peak=bytes_ / t_call / 1e6 / HBM_PEAK_GBS,
        workload=f"windowed prefill, 4 x 8192 tokens from position 0, {heads(model)}, window 128",
        rope=dict(ms=t_rope, bytes=rope_bytes, tokens=T, gbs=rope_bytes / t_rope / 1e6,
                  frac_hbm_peak=rope_bytes / t_rope / 1e6 / HBM_PEAK_GBS,
                  workload=f"RoPE + staging write of 32768 tokens ({heads(model)})"))


def bench_c1(hsw, wl, steps, stream):
    """The fp32 windowed layer (1 x 512 tokens, 4 q / 1 KV head, logits near
    -25, sinks near +1): RoPE + staging write, then the windowed prefill.
    Launch-bound: the time is reported with no roofline claim."""
    d = wl.logit_shift_layer()
    sh = d["shape"]
    T = 512
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    q_rot, kst, vst = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    kring = torch.zeros((1, 1, 128, 192), dtype=torch.float32, device=DEV)
    vring = torch.zeros((1, 1, 128, 128), dtype=torch.float32, device=DEV)
    out = torch.empty((T, 4, 128), dtype=torch.float32, device=DEV)

    def rope(i):
        hsw.hsw_rope_partial_kv_write(sh, T, g["q"], g["k"], g["v"], g["pos"], None, hsw.HSW_DST_STAGING,
                                      kst, vst, T, None, q_rot, None, stream)

    def prefill(i):
        hsw.hsw_swa_prefill(sh, 1, T, g["cu_seqlens"], g["start_pos"], q_rot, kst, vst, kring, vring, g["sinks"],
                            out, stream)
    for i in range(10):
        rope(i)
        prefill(i)
    n = max(steps, 200)
    t_rope = ev_time(rope, n, stream)
    t_pre = ev_time(prefill, n, stream)
    return dict(rope_ms=t_rope, swa_prefill_ms=t_pre, chain_ms=t_rope + t_pre, launches_per_run=n, tokens=T,
                roofline=None, workload="one windowed layer in fp32: 1 x 512 tokens, 4 q / 1 KV head, window 128, "
                                        "sinks, logits near -25 (launch-bound; no roofline claim)")


def bench_copy(steps, stream, nbytes=1 << 30):
    """Plain device-to-device copy of `nbytes` (torch's copy kernel): the
    reference for scaling the HBM byte counters of a profiled run (it reads
    and writes exactly nbytes per launch)."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=DEV).normal_()
    dst = torch.empty_like(src)

    def call(i):
        dst.copy_(src)
    warm(call, stream)
    t = ev_time(call, max(steps, 10), stream)
    return dict(ms=t, bytes=2 * nbytes, gbs=2 * nbytes / t / 1e6, read_bytes=nbytes, write_bytes=nbytes)


def bench_swa_decode(hsw, wl, steps, stream, replicas=8, model=None):
    """Windowed decode, 256 sequences at positions U{128..524288}; 8 replicas
    of (q, rings, out) so each launch reads HBM (working set 178 MB < MALL)."""
    model = model or wl.FLASH
    hq, hkv = model.n_q_heads, model.swa_kv_heads
    S = 256
    reps = []
    for r in range(replicas):
        b = wl.swa_decode_batch(seed=3 if r == 0 else 300 + r, device=DEV, **wl.model_kw(model, "swa"))
        d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in b.items()}
        q_rot = torch.empty_like(d["q"])
        hsw.hsw_rope_partial_kv_write(b["shape"], S, d["q"], d["k"], d["v"], d["pos"], d["seq"],
                                      hsw.HSW_DST_RING, d["kring"], d["vring"], S, None, q_rot, None, stream)
        d["q_rot"] = q_rot
        d["out"] = torch.empty((S, hq, 128), dtype=torch.bfloat16, device=DEV)
        reps.append(d)
    sh = b["shape"]

    def call(i):
        d = reps[i % replicas]
        hsw.hsw_swa_decode(sh, S, d["pos"], d["q_rot"], d["kring"], d["vring"], d["sinks"], d["out"], stream)

    def fused(i):
        d = reps[i % replicas]
        hsw.hsw_swa_decode_qrope(sh, S, d["pos"], d["q"], d["kring"], d["vring"], d["sinks"], d["out"], stream)

    def rope(i):
        d = reps[i % replicas]
        hsw.hsw_rope_partial_kv_write(sh, S, d["q"], d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_RING,
                                      d["kring"], d["vring"], S, None, d["q_rot"], None, stream)

    def rope_kv(i):
        d = reps[i % replicas]
        hsw.hsw_rope_partial_kv_write(sh, S, None, d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_RING,
                                      d["kring"], d["vring"], S, None, None, None, stream)
    for i in range(2 * replicas):
        call(i)
        fused(i)
    warm(call, stream)
    n = max(steps, 25) * replicas
    t = ev_time(call, n, stream)
    t_fused = ev_time(fused, n, stream)
    t_rope = ev_time(rope, n, stream)
    t_rope_kv = ev_time(rope_kv, n, stream)
    bytes_ = S * (hkv * 128 * (192 + 128) * 2 + hq * 192 * 2 + hq * 128 * 2)
    flops = S * hq * 128 * 2 * (192 + 128)
    fused_res = dict(ms=t_fused, gbs=bytes_ / t_fused / 1e6, rope_kv_ms=t_rope_kv, rope_ms=t_rope,
                     chain_ms=t_rope_kv + t_fused, unfused_chain_ms=t_rope + t,
                     workload="K/V-only RoPE into the rings + hsw_swa_decode_qrope (q rotated in the "
                              "kernel, kept in fp32) against RoPE + hsw_swa_decode, same workload")
    floor = bench_stream_floor(steps, stream, model, replicas)
    return dict(ms=t, bytes=bytes_, gbs=bytes_ / t / 1e6, frac_hbm_peak=bytes_ / t / 1e6 / HBM_PEAK_GBS,
                flops=flops, tokens=S, launches=n, replicas=replicas, fused=fused_res,
                stream_floor_ms=floor["ms"], stream_floor_gbs=floor["gbs"],
                time_vs_stream_floor=floor["ms"] / t,
                workload=f"windowed decode, 256 sequences at positions U{{128..524288}}, {heads(model)}, "
                         "128-slot ring")


def measure_lib():
    """libhsw_measure.so: measurement-only kernels (not the attention path)."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hybrid_sliding_window_amd",
                        "libhsw_measure.so")
    lib = ctypes.CDLL(path)
    f = lib.hsw_measure_read_items
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    return lib


def bench_stream_floor(steps, stream, model=None, replicas=8):
    """A plain read (loads only, nothing computed) of the windowed decode's
    input bytes in the decode's layout: per (sequence, KV head) item its 48 KiB
    K ring, 32 KiB V ring and the 3 KiB (Flash; 6 KiB Pro) of its query heads,
    256 sequences, 8 replicas as in the decode's timing.  What the memory
    system delivers for these bytes to the simplest kernel: the decode
    kernel's time is set beside it."""
    from hybrid_sliding_window_amd import workloads as wl
    model = model or wl.FLASH
    hq, hkv = model.n_q_heads, model.swa_kv_heads
    items = 256 * hkv
    kb, vb, qb = 128 * 192 * 2, 128 * 128 * 2, (hq // hkv) * 192 * 2
    lib = measure_lib()
    reps = [tuple(torch.ones(items * n, dtype=torch.uint8, device=DEV) for n in (kb, vb, qb))
            for _ in range(replicas)]
    sink = torch.zeros(1024, dtype=torch.int32, device=DEV)
    sp = stream.cuda_stream

    def call(i):
        k, v, q = reps[i % replicas]
        rc = lib.hsw_measure_read_items(k.data_ptr(), v.data_ptr(), q.data_ptr(), items, kb, vb, qb,
                                        sink.data_ptr(), sp)
        if rc:
            raise RuntimeError(f"hsw_measure_read_items failed ({rc})")
    for i in range(2 * replicas):
        call(i)
    warm(call, stream)
    t = ev_time(call, max(steps, 25) * replicas, stream)
    nbytes = items * (kb + vb + qb)
    return dict(ms=t, bytes=nbytes, gbs=nbytes / t / 1e6, frac_hbm_peak=nbytes / t / 1e6 / HBM_PEAK_GBS,
                workload=f"plain read of the windowed decode's inputs ({items} items of K {kb} B, V {vb} B, "
                         f"q {qb} B), one workgroup per item, loads only")


def bench_full_decode(hsw, wl, steps, stream, model=None):
    """Full-attention decode, 64 sequences, contexts U{32768..131072}, split-K 2048."""
    model = model or wl.FLASH
    hq, hkv = model.n_q_heads, model.full_kv_heads
    b = wl.full_decode_batch(seed=4, device=DEV, **wl.model_kw(model, "full"))
    sh = b["shape"]
    S = 64
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in b.items()}
    rows = d["kpool"].shape[0]
    q_rot = torch.empty_like(d["q"])
    hsw.hsw_rope_partial_kv_write(sh, S, d["q"], d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_POOL,
                                  d["kpool"], d["vpool"], rows, d["seq_base"], q_rot, None, stream)
    max_ctx = int(b["ctx_len"].max())
    wsb = hsw.hsw_full_decode_workspace_bytes(sh, S, max_ctx, 2048)
    ws = torch.empty(wsb // 4 + 4, dtype=torch.float32, device=DEV)
    out = torch.empty((S, hq, 128), dtype=torch.bfloat16, device=DEV)

    def call(i):
        hsw.hsw_full_decode_splitk(sh, S, max_ctx, d["ctx_len"], d["seq_base"], q_rot, d["kpool"], d["vpool"],
                                   rows, None, 2048, ws, wsb, out, stream)
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    n = max(steps // 2, 20)
    t = ev_time(call, n, stream)

    # the fused chain: K/V-only RoPE into the pool, then the decode that
    # rotates q itself (fp32 rotated dims, no q_rot written or read)
    def fused(i):
        hsw.hsw_full_decode_splitk_qrope(sh, S, max_ctx, d["ctx_len"], d["seq_base"], d["q"], d["kpool"],
                                         d["vpool"], rows, None, 2048, ws, wsb, out, stream)

    def rope(i):
        hsw.hsw_rope_partial_kv_write(sh, S, d["q"], d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_POOL,
                                      d["kpool"], d["vpool"], rows, d["seq_base"], q_rot, None, stream)

    def rope_kv(i):
        hsw.hsw_rope_partial_kv_write(sh, S, None, d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_POOL,
                                      d["kpool"], d["vpool"], rows, d["seq_base"], None, None, stream)
    for i in range(3):
        fused(i)
    torch.cuda.synchronize()
    t_fused = ev_time(fused, n, stream)
    t_rope = ev_time(rope, max(steps, 20), stream)
    t_rope_kv = ev_time(rope_kv, max(steps, 20), stream)
    L = int(b["ctx_len"].sum())
    bytes_ = L * hkv * (192 + 128) * 2 + S * hq * (192 + 128) * 2
    flops = L * hq * 2 * (192 + 128)
    del d, ws
    fused_res = dict(ms=t_fused, gbs=bytes_ / t_fused / 1e6, rope_kv_ms=t_rope_kv, rope_ms=t_rope,
                     chain_ms=t_rope_kv + t_fused, unfused_chain_ms=t_rope + t,
                     workload="K/V-only RoPE into the pool + hsw_full_decode_splitk_qrope (q rotated in the "
                              "kernel, kept in fp32) against RoPE + hsw_full_decode_splitk, same workload")
    return dict(ms=t, bytes=bytes_, gbs=bytes_ / t / 1e6, frac_hbm_peak=bytes_ / t / 1e6 / HBM_PEAK_GBS,
                tflops=flops / t / 1e9, flops=flops, tokens=S, launches_per_run=n, fused=fused_res,
                workload=f"full-attention decode, 64 sequences, contexts U{{32768..131072}}, {hq} q / {hkv} KV "
                         "heads, split-K 2048")


def bench_full_prefill(hsw, wl, steps, stream, model=None):
    """Full-attention chunked prefill: 8192 tokens after 131072 prior rows."""
    model = model or wl.FLASH
    hq, hkv = model.n_q_heads, model.full_kv_heads
    b = wl.full_prefill_batch(seed=5, device=DEV, **wl.model_kw(model, "full"))
    sh = b["shape"]
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in b.items()}
    T = 8192
    rows = d["kpool"].shape[0]
    q_rot = torch.empty_like(d["q"])
    hsw.hsw_rope_partial_kv_write(sh, T, d["q"], d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_POOL,
                                  d["kpool"], d["vpool"], rows, d["seq_base"], q_rot, None, stream)
    out = torch.empty((T, hq, 128), dtype=torch.bfloat16, device=DEV)

    def call(i):
        hsw.hsw_full_prefill_chunk(sh, 1, T, d["cu_seqlens"], d["start_pos"], d["seq_base"], q_rot, d["kpool"],
                                   d["vpool"], rows, None, out, stream)
    call(0)
    torch.cuda.synchronize()
    n = max(3, steps // 10)
    t = ev_time(call, n, stream)

    # the fused chain: K/V-only RoPE into the pool, then the prefill that
    # rotates q itself (no q_rot written or read)
    def fused(i):
        hsw.hsw_full_prefill_chunk_qrope(sh, 1, T, d["cu_seqlens"], d["start_pos"], d["seq_base"], d["q"],
                                         d["kpool"], d["vpool"], rows, None, out, stream)

    def rope(i):
        hsw.hsw_rope_partial_kv_write(sh, T, d["q"], d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_POOL,
                                      d["kpool"], d["vpool"], rows, d["seq_base"], q_rot, None, stream)

    def rope_kv(i):
        hsw.hsw_rope_partial_kv_write(sh, T, None, d["k"], d["v"], d["pos"], d["seq"], hsw.HSW_DST_POOL,
                                      d["kpool"], d["vpool"], rows, d["seq_base"], None, None, stream)
    fused(0)
    torch.cuda.synchronize()
    t_fused = ev_time(fused, n, stream)
    t_rope = ev_time(rope, max(steps, 20), stream)
    t_rope_kv = ev_time(rope_kv, max(steps, 20), stream)
    pairs = T * 131072 + T * (T + 1) // 2
    flops = pairs * hq * 2 * (192 + 128)
    fused_res = dict(ms=t_fused, tflops=flops / t_fused / 1e9, rope_kv_ms=t_rope_kv, rope_ms=t_rope,
                     chain_ms=t_rope_kv + t_fused, unfused_chain_ms=t_rope + t,
                     workload="K/V-only RoPE into the pool + hsw_full_prefill_chunk_qrope (q rotated in the "
                              "kernel) against RoPE + hsw_full_prefill_chunk, same workload")
    return dict(ms=t, flops=flops, tflops=flops / t / 1e9, frac_mfma_peak=flops / t / 1e9 / BF16_PEAK_TFLOPS,
                tokens=T, launches_per_run=n, fused=fused_res,
                workload=f"full-attention prefill, 8192 tokens after 131072 prior rows, {hq} q / {hkv} KV heads")


def bench_kvm_snapshot(hsw, wl, steps, stream, model=None):
    """Ring snapshot and restore of one sequence (hsw_kvm_snapshot /
    hsw_kvm_restore): every windowed layer's ring block (model's windowed
    layers, 128 slots, K and V) copied out to a snapshot slot and back, on
    rings of 129 sequences per layer."""
    model = model or wl.FLASH
    n_swa = model.n_layers - model.n_full
    hkv = model.swa_kv_heads
    S = 129
    k = [torch.empty((S, hkv, 128, 192), dtype=torch.bfloat16, device=DEV) for _ in range(n_swa)]
    v = [torch.empty((S, hkv, 128, 128), dtype=torch.bfloat16, device=DEV) for _ in range(n_swa)]
    cfg = hsw.KvmConfig(n_swa, hkv, 128, 192, 128, 2, S, 1 << 20, 2)
    sb = hsw.hsw_kvm_snapshot_bytes(cfg)
    snap_buf = torch.empty((2 * sb // 2,), dtype=torch.bfloat16, device=DEV)
    kv = hsw.KvManager(cfg, k, v, snap_buf)
    seq, _ = kv.admit(1024)
    kv.append(seq, [1, 2, 3])
    sid = kv.snapshot(seq, stream)
    warm(lambda i: kv.restore(sid, stream), stream)
    n = max(steps, 20)
    t_restore = ev_time(lambda i: kv.restore(sid, stream), n, stream)
    t_snap = ev_time(lambda i: _snap_cycle(kv, seq, stream), n, stream)
    kv.close()
    del k, v, snap_buf
    return dict(ms=t_snap, restore_ms=t_restore, bytes=2 * sb, gbs=2 * sb / t_snap / 1e6,
                restore_gbs=2 * sb / t_restore / 1e6, snapshot_bytes=sb,
                workload=f"ring snapshot of one sequence, {n_swa} windowed layers x {hkv} KV heads x 128 slots x "
                         f"(192 + 128) bf16 ({sb / 1e6:.1f} MB each way)")


def bench_vit(hsw, wl, steps, stream, parts=("window", "full", "rope", "window_rope")):
    """Vision-encoder attention on 16 pictures of 64 x 64 patches (65536
    tokens, 16 q / 4 KV heads of width 64): a window block (column order of
    the merge units, the sink key), a full block, and the 2D RoPE of q and k.
    Two replicas of the inputs alternate, so the 0.34 GB a window block
    moves is read from HBM rather than the 256 MB Infinity Cache."""
    grids = wl.VIT_BENCH_GRIDS
    lens = [h * w for h, w in grids]
    T, S, hq, hkv = sum(lens), len(grids), 16, 4
    order = np.concatenate([hsw.hsw_vit_layout(h, w)[2] for h, w in grids]).astype(np.int32)
    rowcol = [np.concatenate([hsw.hsw_vit_layout(h, w)[i] for h, w in grids]) for i in (0, 1)]
    d_order = torch.from_numpy(order).to(DEV)
    d_row, d_col = (torch.from_numpy(x).to(DEV) for x in rowcol)
    reps = []
    for r in range(2):
        b = wl.vit_batch(seed=40 + r, grids=grids, device=DEV)
        b["out"] = torch.empty((T, hq, 64), dtype=torch.bfloat16, device=DEV)
        b["qr"], b["kr"] = torch.empty_like(b["q"]), torch.empty_like(b["k"])
        b["cu"] = b["cu_seqlens"].to(DEV)
        reps.append(b)
    win, full = wl.vit_shape(hq, hkv, 64), wl.vit_shape(hq, hkv, 0)
    maxlen = max(lens)

    def window_call(i):
        b = reps[i % 2]
        hsw.hsw_vit_attention(win, S, maxlen, b["cu"], d_order, 1, b["q"], b["k"], b["v"], None, b["out"], stream)

    def full_call(i):
        b = reps[i % 2]
        hsw.hsw_vit_attention(full, S, maxlen, b["cu"], None, 0, b["q"], b["k"], b["v"], None, b["out"], stream)

    def rope_call(i):
        b = reps[i % 2]
        hsw.hsw_vit_rope_2d(win, T, b["q"], b["k"], d_row, d_col, b["qr"], b["kr"], stream)

    def window_rope_call(i):   # the 2D RoPE fused into the window block (unrotated q, k)
        b = reps[i % 2]
        hsw.hsw_vit_window_attention_rope(win, S, maxlen, b["cu"], d_order, 1, d_row, d_col, b["q"], b["k"],
                                          b["v"], None, b["out"], stream)
    res = {"window": float("nan"), "full": float("nan"), "rope": float("nan"), "window_rope": float("nan")}
    for name, fn, n in (("window", window_call, max(steps, 20) * 2), ("full", full_call, max(steps // 5, 4)),
                        ("rope", rope_call, max(steps, 20) * 2), ("window_rope", window_rope_call, max(steps, 20) * 2)):
        if name not in parts:
            continue
        fn(0)
        fn(1)
        warm(fn, stream)
        res[name] = ev_time(fn, n, stream)
    # algorithmic bytes / flops
    tok_bytes = (2 * hq * 64 + 2 * hkv * 64) * 2            # q, out; k, v (bf16)
    win_pairs = 0
    for n in lens:
        for lo in range(0, n, 64):
            nw = min(64, n - lo)
            win_pairs += nw * (nw + (1 if lo > 0 else 0))
    full_pairs = sum(n * n for n in lens)
    win_bytes = T * tok_bytes
    win_flops = win_pairs * hq * 64 * 4
    full_flops = full_pairs * hq * 64 * 4
    rope_bytes = T * (hq + hkv) * 64 * 2 * 2
    return dict(window=dict(ms=res["window"], bytes=win_bytes, gbs=win_bytes / res["window"] / 1e6,
                            traffic=measured_traffic("vit_window"),
                            frac_hbm_peak=win_bytes / res["window"] / 1e6 / HBM_PEAK_GBS,
                            tflops=win_flops / res["window"] / 1e9, flops=win_flops, tokens=T,
                            workload="window block: 64-token windows in column order of the merge units + "
                                     "the sink key"),
                full=dict(ms=res["full"], flops=full_flops, tflops=full_flops / res["full"] / 1e9, tokens=T,
                          frac_mfma_peak=full_flops / res["full"] / 1e9 / BF16_PEAK_TFLOPS,
                          workload="full block: every picture attends to itself"),
                rope=dict(ms=res["rope"], bytes=rope_bytes, gbs=rope_bytes / res["rope"] / 1e6, tokens=T,
                          workload="2D RoPE of q and k"),
                window_rope=dict(ms=res["window_rope"], bytes=win_bytes, gbs=win_bytes / res["window_rope"] / 1e6,
                                 frac_hbm_peak=win_bytes / res["window_rope"] / 1e6 / HBM_PEAK_GBS, tokens=T,
                                 chain_ms=res["window_rope"], unfused_chain_ms=res["rope"] + res["window"],
                                 workload="window block with the 2D RoPE fused (hsw_vit_window_attention_rope, "
                                          "unrotated q and k) against 2D RoPE + window block"),
                workload=f"vision encoder, {S} pictures of 64 x 64 patches ({T} tokens), {hq} q / {hkv} KV "
                         "heads of width 64")


def _snap_cycle(kv, seq, stream):
    kv.drop_snapshot(kv.snapshot(seq, stream))


def bench_hybrid(hsw, wl, steps, stream, model=None):
    """One hybrid step (hybrid_sliding_window_amd.hybrid.HybridStep) over the
    model's attention-only layers (Flash: 39 windowed + 9 full, Pro: 60 + 10,
    full layers at seeded indices), each running RoPE + prefill for an
    8192-token chunk at positions 131072..139263 and RoPE + decode for 128
    sequences with contexts U{4096..262144}."""
    from hybrid_sliding_window_amd.hybrid import HybridStep
    model = model or wl.FLASH
    hs = HybridStep(hsw, device=DEV, model=model)
    hs.step(stream)
    torch.cuda.synchronize()
    # the step as the metric defines it: 5 runs of n >= 3 steps, median
    n = max(3, steps)
    runs = []
    t = ev_time(lambda i: hs.step(stream), n, stream, runs)
    # variants, 3 runs of one step each: every attention call rotating q
    # itself; decode calls on a second stream beside the prefill calls
    # (fused q-RoPE on, then off)
    hs.qrope = True
    hs.step(stream)
    torch.cuda.synchronize()
    t_q = ev_time(lambda i: hs.step(stream), 1, stream, reps=3)
    hs.step(stream, overlap=True)
    torch.cuda.synchronize()
    t_qo = ev_time(lambda i: hs.step(stream, overlap=True), 1, stream, reps=3)
    hs.qrope = False
    hs.step(stream, overlap=True)
    torch.cuda.synchronize()
    t_o = ev_time(lambda i: hs.step(stream, overlap=True), 1, stream, reps=3)
    timer = []
    hs.step(stream, timer)
    torch.cuda.synchronize()
    kinds = {"rope": 0.0, "swa_prefill": 0.0, "swa_decode": 0.0, "full_prefill": 0.0, "full_decode": 0.0}
    for kind, e0, e1 in timer:
        kinds[kind] += e0.elapsed_time(e1)
    T, S = hs.T, hs.S
    nl, nf = len(hs.pattern), len(hs.pattern) - sum(hs.pattern)
    res = dict(ms=t, tokens_per_s=(T + S) / (t / 1e3), steps_per_run=n, runs_ms=runs,
               per_call_ms={k: round(v, 3) for k, v in kinds.items()},
               qrope_ms=t_q, qrope_tokens_per_s=(T + S) / (t_q / 1e3),
               overlap_ms=t_o, overlap_tokens_per_s=(T + S) / (t_o / 1e3),
               qrope_overlap_ms=t_qo, qrope_overlap_tokens_per_s=(T + S) / (t_qo / 1e3),
               layers=f"{nl - nf} windowed + {nf} full (seeded pattern)", pool_gb=round(hs.pool_gb, 1),
               workload=f"hybrid step {model.name}: {nl} layers, 8192-token chunk at 131072 + 128 decode "
                        "sequences U{4096..262144}")
    del hs
    return res


def own_roofline(d):
    """Add the call's own roofline fraction t_floor / t, t_floor =
    max(flops / dense bf16 MFMA peak, bytes / HBM peak) over the algorithmic
    work it reports, and tokens/s where it reports a token count."""
    if not isinstance(d, dict) or not d.get("ms") or d["ms"] != d["ms"]:
        return d
    t = d["ms"] / 1e3
    floors = {}
    if d.get("flops"):
        floors["mfma"] = d["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    if d.get("bytes"):
        floors["hbm"] = d["bytes"] / (HBM_PEAK_GBS * 1e9)
    if floors:
        bound = max(floors, key=floors.get)
        d["roofline_bound"] = bound
        d["roofline_frac"] = floors[bound] / t
    if d.get("tokens"):
        d["tokens_per_s"] = d["tokens"] / t
    return d


def rounded(d):
    d = own_roofline(dict(d))
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def bench_pro(hsw, wl, args, stream):
    """Every call of the path and the 70-layer hybrid step at MiMo-V2.6-Pro
    shapes (128 q heads, 8 KV heads on both layer kinds, value scale 0.612)."""
    m = wl.PRO
    out = {"model": m.name, "heads": "128 q / 8 KV heads on both layer kinds", "value_scale": m.value_scale}
    pre = bench_swa_prefill(hsw, wl, args.steps, args.warmup, stream, m)
    print(f"[bench] pro swa_prefill {pre['ms']:.3f} ms {pre['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    out["rope_partial_kv_write"] = rounded(pre.pop("rope"))
    out["swa_prefill_qrope"] = rounded(pre.pop("fused"))
    out["swa_prefill"] = rounded(pre)
    torch.cuda.empty_cache()
    dec = bench_swa_decode(hsw, wl, args.steps, stream, model=m)
    print(f"[bench] pro swa_decode {dec['ms'] * 1e3:.1f} us {dec['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    out["swa_decode_qrope"] = rounded(dec.pop("fused"))
    out["swa_decode"] = rounded(dec)
    torch.cuda.empty_cache()
    fd = bench_full_decode(hsw, wl, args.steps, stream, m)
    print(f"[bench] pro full_decode {fd['ms']:.3f} ms {fd['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    out["full_decode_splitk_qrope"] = rounded(fd.pop("fused"))
    out["full_decode_splitk"] = rounded(fd)
    torch.cuda.empty_cache()
    fp = bench_full_prefill(hsw, wl, args.steps, stream, m)
    print(f"[bench] pro full_prefill {fp['ms']:.2f} ms {fp['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    out["full_prefill_chunk_qrope"] = rounded(fp.pop("fused"))
    out["full_prefill_chunk"] = rounded(fp)
    torch.cuda.empty_cache()
    hy = bench_hybrid(hsw, wl, args.steps // 25, stream, m)
    print(f"[bench] pro hybrid step {hy['ms']:.1f} ms {hy['tokens_per_s']:.0f} tok/s {hy['per_call_ms']}; "
          f"fused q-RoPE step {hy['qrope_ms']:.1f} ms; decode on a second stream {hy['overlap_ms']:.1f} ms "
          f"(fused {hy['qrope_overlap_ms']:.1f} ms)",
          file=sys.stderr, flush=True)
    out["hybrid_step"] = rounded(hy)
    torch.cuda.empty_cache()
    return out


def cpu_oracle_protocol(seed=2024):
    """The fp64 oracle on the host cores (attention only; input generation,
    seeded and synthetic, is untimed): workloads 1-4 in full, and the hybrid
    step on a sample (32 chunk rows of one full layer, 256 of one windowed
    layer, 8 of the 128 decodes of each kind) extrapolated linearly by row
    count to its 39 + 9 layers and labelled "extrapolated".  Reported as a
    baseline only."""
    import oracle
    from hybrid_sliding_window_amd import workloads as wl
    rng = np.random.default_rng(seed)
    tau, lam = 1 / math.sqrt(192), 0.707
    gen_s = [0.0]

    def normal(*shape, out=None):
        """N(0, 1) in fp64, drawn into `out` when given (large arrays are
        allocated once and redrawn in place)."""
        t0 = time.perf_counter()
        a = rng.standard_normal(None if out is not None else shape, dtype=np.float64, out=out)
        gen_s[0] += time.perf_counter() - t0
        return a

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def entry(sec, flops, what):
        print(f"[bench] cpu oracle: {what}: {sec:.2f} s", file=sys.stderr, flush=True)
        return dict(seconds=round(sec, 3), flops=flops, tflops=flops / sec / 1e12, workload=what)

    res = {}
    # 1: the fp32 windowed layer, RoPE + windowed attention
    d = wl.logit_shift_layer()
    P1 = d["pos"].numpy()
    q1, k1, v1, s1 = (d[x].double().numpy() for x in ("q", "k", "v", "sinks"))
    sec = timed(lambda: oracle.attn_linear(oracle.rope(q1, P1, 1e4), P1, oracle.rope(k1, P1, 1e4), v1, 0,
                                           window=128, tau=tau, lam=lam, sinks=s1))
    res["c1"] = entry(sec, swa_prefill_pairs([512], [0]) * 4 * 2 * 320, "1 x 512 tokens, 4 q / 1 KV head, window 128")
    # 2: windowed prefill, 4 x 8192 tokens, 64 q / 8 KV heads
    sinks = 1.0 + 0.25 * normal(64)
    pos = np.arange(8192)
    sec = 0.0
    q, k, v = np.empty((8192, 64, 192)), np.empty((8192, 8, 192)), np.empty((8192, 8, 128))
    for _ in range(4):
        normal(out=q), normal(out=k), normal(out=v)
        sec += timed(lambda: oracle.attn_linear(q, pos, k, v, 0, window=128, tau=tau, lam=lam, sinks=sinks))
    del q, k, v
    res["c2"] = entry(sec, 4 * swa_prefill_pairs([8192], [0]) * 64 * 2 * 320,
                      "4 x 8192 tokens from position 0, 64 q / 8 KV heads, window 128, sinks")
    # 3: windowed decode, 256 sequences over full 128-slot rings
    P3 = rng.integers(128, 524289, size=256)
    q, kr, vr = normal(256, 64, 192), normal(256, 8, 128, 192), normal(256, 8, 128, 128)
    sec = timed(lambda: oracle.ring_decode(q, P3, kr, vr, tau=tau, lam=lam, sinks=sinks))
    del kr, vr
    res["c3"] = entry(sec, 256 * 64 * 128 * 2 * 320, "256 sequences at positions U{128..524288}, 64 q / 8 KV heads")
    # one pool of 262144 rows (4 KV heads) serves the full-attention contexts:
    # each sequence reads its own prefix of it (the work depends only on the
    # lengths)
    kp, vp = normal(262144, 4, 192), normal(262144, 4, 128)
    # 4: full decode, 64 sequences, contexts U{32768..131072}
    L4 = rng.integers(32768, 131073, size=64)
    q = normal(64, 64, 192)
    sec = sum(timed(lambda s=s: oracle.attn_linear(q[s:s + 1], np.array([L4[s] - 1]), kp[:L4[s]], vp[:L4[s]], 0,
                                                   window=0, tau=tau, lam=lam)) for s in range(64))
    res["c4"] = entry(sec, int(L4.sum()) * 64 * 2 * 320, "64 sequences, contexts U{32768..131072}, 64 q / 4 KV heads")
    # 5: sampled, then extrapolated by row count
    rows = np.sort(rng.choice(8192, 32, replace=False))
    qf = normal(32, 64, 192)
    t_fp = timed(lambda: oracle.attn_linear(qf, 131072 + rows, kp[:139264], vp[:139264], 0, window=0, tau=tau,
                                            lam=lam))
    qw, kw, vw = normal(256, 64, 192), normal(256 + 127, 8, 192), normal(256 + 127, 8, 128)
    t_wp = timed(lambda: oracle.attn_linear(qw, 131072 + np.arange(256), kw, vw, 131072 - 127, window=128, tau=tau,
                                            lam=lam, sinks=sinks))
    L5 = rng.integers(4096, 262145, size=8)
    qd = normal(8, 64, 192)
    t_fd = sum(timed(lambda s=s: oracle.attn_linear(qd[s:s + 1], np.array([L5[s] - 1]), kp[:L5[s]], vp[:L5[s]], 0,
                                                    window=0, tau=tau, lam=lam)) for s in range(8))
    qr_, kr_, vr_ = normal(8, 64, 192), normal(8, 8, 128, 192), normal(8, 8, 128, 128)
    t_wd = timed(lambda: oracle.ring_decode(qr_, rng.integers(4096, 262145, size=8), kr_, vr_, tau=tau, lam=lam,
                                            sinks=sinks))
    del kp, vp
    print(f"[bench] cpu oracle: hybrid-step sample {t_fp + t_wp + t_fd + t_wd:.2f} s", file=sys.stderr, flush=True)
    ext = t_fp * (8192 / 32) * 9 + t_wp * (8192 / 256) * 39 + t_fd * (128 / 8) * 9 + t_wd * (128 / 8) * 39
    res["c5"] = dict(label="extrapolated", seconds=round(ext, 1),
                     sampled_seconds=round(t_fp + t_wp + t_fd + t_wd, 3),
                     sample="32 of the 8192 chunk rows of one full layer (131072 prior rows), 256 of one windowed "
                            "layer, 8 of the 128 decode sequences of each kind; scaled by row count to 9 full + 39 "
                            "windowed layers",
                     workload="hybrid step, 48 layers: 8192-token chunk at 131072 + 128 decode sequences")
    for v in res.values():
        if "tflops" in v:
            v["tflops"] = round(v["tflops"], 6)
    return dict(configs=res, cores=oracle.num_threads(), host=host_cpu(), kind="oracle",
                input_generation_seconds=round(gen_s[0], 1),
                note="fp64 oracle, attention only (input generation untimed); a baseline, not a target")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--quick", action="store_true", help="only the two metric calls")
    ap.add_argument("--only", choices=["swa_prefill", "swa_decode", "full_decode", "full_prefill", "hybrid", "copy",
                                       "kvm_snapshot", "vit", "stream"],
                    help="run one call's timing only (for profiling) and print its numbers")
    ap.add_argument("--model", choices=["flash", "pro"], default="flash", help="shapes for --only")
    ap.add_argument("--vit-part", choices=["all", "window", "full", "rope", "window_rope"], default="all",
                    help="with --only vit: time one of the vision-encoder calls only (for profiling)")
    ap.add_argument("--no-pro", action="store_true", help="skip the MiMo-V2.6-Pro section")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the attention core is measured on one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by sequence / KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    from hybrid_sliding_window_amd import hsw
    from hybrid_sliding_window_amd import workloads as wl
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.only:
        m = wl.MODELS[args.model]
        fn = {"swa_prefill": lambda: bench_swa_prefill(hsw, wl, args.steps, args.warmup, stream, m),
              "swa_decode": lambda: bench_swa_decode(hsw, wl, args.steps, stream, model=m),
              "full_decode": lambda: bench_full_decode(hsw, wl, args.steps, stream, m),
              "full_prefill": lambda: bench_full_prefill(hsw, wl, args.steps, stream, m),
              "hybrid": lambda: bench_hybrid(hsw, wl, args.steps // 25, stream, m),
              "copy": lambda: bench_copy(args.steps, stream),
              "stream": lambda: bench_stream_floor(args.steps, stream, m),
              "kvm_snapshot": lambda: bench_kvm_snapshot(hsw, wl, args.steps, stream, m),
              "vit": lambda: bench_vit(hsw, wl, args.steps, stream,
                                       ("window", "full", "rope", "window_rope") if args.vit_part == "all"
                                       else (args.vit_part,))}[
            args.only]
        r = fn()
        print(json.dumps({"only": args.only, "model": m.name,
                          **{k: v for k, v in r.items() if not isinstance(v, dict) or k in ("fused", "window", "full",
                                                                                            "rope", "window_rope")}}))
        return

    pre = bench_swa_prefill(hsw, wl, args.steps, args.warmup, stream)
    clocks = {"after_windowed_prefill": gpu_clocks_power()}
    print(f"[bench] swa_prefill {pre['ms']:.3f} ms {pre['tflops']:.1f} TFLOP/s {pre['gbs']:.0f} GB/s; fused q-RoPE "
          f"{pre['fused']['ms']:.3f} ms, chain {pre['fused']['chain_ms']:.3f} vs {pre['fused']['unfused_chain_ms']:.3f} ms",
          file=sys.stderr, flush=True)
    dec = bench_swa_decode(hsw, wl, args.steps, stream)
    print(f"[bench] swa_decode {dec['ms'] * 1e3:.1f} us {dec['gbs']:.0f} GB/s (a plain read of its inputs: "
          f"{dec['stream_floor_ms'] * 1e3:.1f} us); fused q-RoPE "
          f"{dec['fused']['ms'] * 1e3:.1f} us, chain {dec['fused']['chain_ms'] * 1e3:.1f} vs "
          f"{dec['fused']['unfused_chain_ms'] * 1e3:.1f} us", file=sys.stderr, flush=True)
    torch.cuda.empty_cache()
    calls = {"rope_partial_kv_write": pre.pop("rope"), "swa_prefill_qrope": pre.pop("fused"),
             "swa_decode_qrope": dec.pop("fused"), "swa_decode": dec,
             "fp32_windowed_layer": bench_c1(hsw, wl, args.steps, stream)}
    if not args.quick:
        fd = bench_full_decode(hsw, wl, args.steps, stream)
        print(f"[bench] full_decode {fd['ms']:.3f} ms {fd['gbs']:.0f} GB/s; fused q-RoPE {fd['fused']['ms']:.3f} ms, "
              f"chain {fd['fused']['chain_ms']:.3f} vs {fd['fused']['unfused_chain_ms']:.3f} ms",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        fp = bench_full_prefill(hsw, wl, args.steps, stream)
        print(f"[bench] full_prefill {fp['ms']:.2f} ms {fp['tflops']:.1f} TFLOP/s; fused q-RoPE "
              f"{fp['fused']['ms']:.2f} ms, chain {fp['fused']['chain_ms']:.2f} vs "
              f"{fp['fused']['unfused_chain_ms']:.2f} ms", file=sys.stderr, flush=True)
        calls["full_decode_splitk_qrope"] = fd.pop("fused")
        calls["full_decode_splitk"] = fd
        calls["full_prefill_chunk_qrope"] = fp.pop("fused")
        calls["full_prefill_chunk"] = fp
        del fd, fp
        torch.cuda.empty_cache()
        snap = bench_kvm_snapshot(hsw, wl, args.steps, stream)
        print(f"[bench] kvm snapshot {snap['ms'] * 1e3:.1f} us restore {snap['restore_ms'] * 1e3:.1f} us "
              f"({snap['gbs']:.0f} / {snap['restore_gbs']:.0f} GB/s)", file=sys.stderr, flush=True)
        calls["kvm_snapshot"] = snap
        torch.cuda.empty_cache()
        vit = bench_vit(hsw, wl, args.steps, stream)
        print(f"[bench] vit window {vit['window']['ms'] * 1e3:.1f} us {vit['window']['gbs']:.0f} GB/s; full "
              f"{vit['full']['ms']:.3f} ms {vit['full']['tflops']:.1f} TFLOP/s; rope {vit['rope']['ms'] * 1e3:.1f} us "
              f"{vit['rope']['gbs']:.0f} GB/s; window with the RoPE fused {vit['window_rope']['ms'] * 1e3:.1f} us",
              file=sys.stderr, flush=True)
        calls["vit"] = vit
        torch.cuda.empty_cache()
        hy = bench_hybrid(hsw, wl, args.steps // 25, stream)
        print(f"[bench] hybrid step {hy['ms']:.1f} ms {hy['tokens_per_s']:.0f} tok/s {hy['per_call_ms']}; "
              f"fused q-RoPE step {hy['qrope_ms']:.1f} ms; decode on a second stream {hy['overlap_ms']:.1f} ms "
              f"(fused {hy['qrope_overlap_ms']:.1f} ms)",
              file=sys.stderr, flush=True)
        calls["hybrid_step"] = hy
        clocks["after_hybrid_step"] = gpu_clocks_power()
        torch.cuda.empty_cache()
    calls["swa_prefill"] = dict(ms=pre["ms"], runs_ms=pre["runs_ms"], launches_per_run=pre["launches_per_run"],
                                tflops=pre["tflops"], gbs=pre["gbs"],
                                frac_mfma_peak=pre["tflops"] / BF16_PEAK_TFLOPS,
                                frac_hbm_peak=pre["gbs"] / HBM_PEAK_GBS, flops=pre["flops"], bytes=pre["bytes"],
                                tokens=4 * 8192)
    for v in calls.values():
        own_roofline(v)
        if isinstance(v, dict):
            for vv in v.values():
                own_roofline(vv)
    line = {
        "metric": METRIC,
        "value": round(pre["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "windowed (SWA) prefill bf16: 4 sequences x 8192 tokens from position 0, "
                               "64 q / 8 KV heads, q/k 192, v 128, window 128, per-head sinks, value scale 0.707",
                   "global_batch": 4, "seq_len": 8192, "parallelism": "single GPU"},
        "swa_decode": {"value": round(dec["gbs"], 1), "unit": "GB/s",
                       "frac_hbm_peak": round(dec["frac_hbm_peak"], 4), "us_per_call": round(dec["ms"] * 1e3, 2),
                       "stream_floor_us": round(dec["stream_floor_ms"] * 1e3, 2),
                       "time_vs_stream_floor": round(dec["time_vs_stream_floor"], 4),
                       "traffic": measured_traffic("swa_decode"),
                       "workload": dec["workload"]},
        "swa_prefill_frac_mfma_peak": round(pre["tflops"] / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(pre["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(pre["gbs"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic("swa_prefill"),
                     "kernel": "hsw_swa_prefill call (sweep kernel + ring commit), 1.513 GB algorithmic per call"},
        "timing": {"statistic": f"median of {RUNS} runs, each of N back-to-back launches between two HIP events",
                   "runs_ms": [round(x, 5) for x in pre["runs_ms"]], "launches_per_run": pre["launches_per_run"]},
        "calls": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                  for k, v in calls.items()},
        "gpu_clocks_power": clocks,
        "host_cpu": host_cpu(),
    }
    if not args.quick and not args.no_pro:
        line["pro"] = bench_pro(hsw, wl, args, stream)
    if not args.no_cpu:
        prot = cpu_oracle_protocol()
        c2 = prot["configs"]["c2"]
        line["cpu_baseline"] = dict(value=c2["tflops"], unit="TFLOP/s", cores=prot["cores"], kind="oracle",
                                    seconds=c2["seconds"],
                                    sample="the windowed-prefill workload in full (4 x 8192 tokens, 64 q / 8 KV "
                                           "heads, window 128, sinks) through the fp64 oracle; algorithmic "
                                           "in-window flops per second")
        line["cpu_oracle"] = prot
    print(json.dumps(line))


if __name__ == "__main__":
    main()
