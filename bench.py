#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path on synthetic inputs already resident in HBM:
  * forward (causal, with LSE) and backward (recompute) on the training workload
    B=2, H=16, N=4096, d=128, bf16 — the attention shape whose FLOP rate is the metric;
  * single-token grouped-query decode: batch 64, Hq=32, Hkv=8, d=128, KV cache L=8192, bf16.

Reported value: forward+backward TFLOP/s with the algorithmic count 4 N^2 d per head
(halved for causal) for the forward and 2.5x that for the backward.  Decode is reported as
algorithmic HBM GB/s (K + V + Q + O + LSE bytes).  Phase times come from HIP events on the
stream the kernels run on, over K steps after 0.3 s of untimed steps and then W untimed
warm-up steps (default 50): after an idle gap the shader clock needs some 25 ms of load to
settle, and the timed steps should not include that ramp.  The fp64 CPU oracle is timed beside
it on a bounded sample.

Secondary lines, each timed on its own after the step (skipped with --no-extras):
  * the other workload configurations: the tiny fp32 forward (B=1 H=1 N=256 d=64), the batched
    d=64 prefill (B=4 H=16 N=1024, causal, with LSE; memory-side roofline) and the long-prefill
    sweep (B=1 H=32 d=128, Q and K x2, N = 4096 / 8192 / 16384, causal and not);
  * decode with per-sequence cache lengths, multi-token decode, chunked prefill (Nq != Nk),
    packed sequences of different lengths (forward and backward), a block-sparse mask (forward
    and backward), a grouped-query training step (B=1 Hq=32 Hkv=8 N=4096 d=128, causal).
FLOP counts are 4 d per (query, key) pair the mask keeps.  Each line carries its fraction of
the roofline: dense bf16 MFMA peak 2516.6 TFLOP/s (256 CUs x 2.4 GHz x 4096 FLOP per clock), HBM
8000 GB/s (the published MI355X figures).

Calibration modes (no step): --copy-calibration runs plain 1 GiB device copies (the reference
for rocprofv3's FETCH_SIZE / WRITE_SIZE byte counters); --stream-read times a streaming read of
a 4 GiB buffer (libexact_calib.so) at several grid sizes, the HBM read rate a kernel that only
reads reaches on this GPU; --mfma-ceiling times a plain loop of dense bf16 MFMAs on every SIMD
and reads the shader clock it runs at (the matrix-core rate such a loop reaches on this GPU);
--atomic-add times fp32 atomic adds in 64 x 128 tiles into a dQ-sized accumulator (the rate a
backward that summed dQ with atomics would depend on).  --prefill-d64, --prefill-d64-sweep and
--tiny-f32 time only the batched d=64 prefill (or the causal d=64 forward over N = 128 .. 1024)
or the tiny fp32 forward, for a profile of its kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
                       [--copy-calibration | --stream-read | --mfma-ceiling | --atomic-add |
                        --prefill-d64 | --prefill-d64-sweep | --tiny-f32]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clock
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def flops_fwd(B, H, N, d, causal):
    f = 4.0 * B * H * N * N * d
    return f * 0.5 if causal else f


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_io_aware_71_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, digest):
    """Per-launch HBM bytes that rocprofv3 counters measured for `kernel`, if they were taken
    on the current kernel source; else None.  The summary file holds one line per kernel:
    `traffic <kernel> digest=<hex> bytes_per_launch=<int> ...`."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        parts = line.split()
        if len(parts) < 3 or parts[0] != "traffic" or parts[1] != kernel:
            continue
        kv = dict(p.split("=", 1) for p in parts[2:] if "=" in p)
        if kv.get("digest") == digest and "bytes_per_launch" in kv:
            return int(kv["bytes_per_launch"])
    return None


def blas_threads():
    """Threads the oracle's BLAS actually runs with, as the BLAS library reports it."""
    try:
        import numpy  # noqa: F401  (threadpoolctl reports only libraries already loaded)
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"]), info[0].get("internal_api", "blas")
    except ImportError:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_baseline(budget_s=15.0):
    """fp64 oracle forward+backward on whole heads of the training workload's shape
    (N=4096, d=128, causal), one head at a time until the time budget is spent or as many
    heads as the workload has were done; scaled to TFLOP/s with the same algorithmic count."""
    import numpy as np
    import oracle
    from synth import default_scale, make_prefill
    B, H, N, d = 2, 16, 4096, 128
    scale = default_scale(d)
    inp = make_prefill(1, 1, 1, N, d, "bf16", seed=1004, with_dout=True)
    heads, t_total = 0, 0.0
    while t_total < budget_s and heads < B * H:
        t0 = time.perf_counter()
        oracle.forward(inp["q"], inp["k"], inp["v"], scale, True)
        oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], scale, True)
        t_total += time.perf_counter() - t0
        heads += 1
    flops = heads * 3.5 * flops_fwd(1, 1, N, d, True)
    threads, blas = blas_threads()
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{heads} passes over one synthetic head (N={N}, d={d}, causal, seed 1004) of the "
                      f"training workload's shape: fp64 forward + backward materialising S and P, "
                      f"{t_total:.1f} s on {threads} {blas} threads "
                      f"({len(os.sched_getaffinity(0))} host cores visible)"}


def copy_calibration(nbytes=1 << 30, reps=5):
    """Plain device-to-device copies of a known size, for scaling rocprofv3's FETCH_SIZE /
    WRITE_SIZE counters to bytes (each copy reads and writes `nbytes`)."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def atomic_add(heads=32, N=4096, reps=16):
    """fp32 atomic adds of 64 x 128 tiles into a [heads, N, 128] fp32 accumulator (the dQ of the
    training workload's shape) with the calibration kernel at two grid sizes: GB/s of added
    floats (4 bytes each) per grid, median of 5 timed launches after 100 ms of warm-up."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_71_amd", "libexact_calib.so"))
    lib.calib_atomic_add.restype = ctypes.c_int
    lib.calib_atomic_add.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    acc = torch.zeros(heads * N * 128, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for blocks in (1024, 4096):
        def run():
            rc = lib.calib_atomic_add(acc.data_ptr(), heads, N, reps, blocks, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"calib_atomic_add failed ({rc})")
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.1:
            run()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[2]
        res[blocks] = blocks * reps * 64 * 128 * 4 / (ms * 1e-3) / 1e9
    print(json.dumps({"atomic_add_fp32_GBps_by_workgroups": res, "tile": "64 x 128 fp32", "tiles_per_workgroup": reps,
                      "accumulator": f"[{heads}, {N}, 128] fp32"}))


def stream_read(nbytes=4 << 30):
    """Streaming read of a device buffer with the calibration kernel at several grid sizes:
    GB/s per grid (median of 5 timed batches of 10 reads, after 200 ms of warm-up reads)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_71_amd", "libexact_calib.so"))
    lib.calib_stream_read.restype = ctypes.c_int
    lib.calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    buf.fill_(3)
    out = torch.empty(1 << 16, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for blocks in (2048, 4096, 8192, 16384, 32768):
        def run():
            rc = lib.calib_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"calib_stream_read failed ({rc})")
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            run()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 10)
        ms = sorted(times)[2]
        res[blocks] = nbytes / (ms * 1e-3) / 1e9
    best = max(res, key=res.get)
    print(json.dumps({"stream_read_bytes": nbytes, "GBps_by_workgroups": res, "best_GBps": res[best],
                      "best_workgroups": best}))


def mfma_ceiling(blocks=1024, iters=4096):
    """Dense bf16 matrix-core rate of a plain loop (four workgroups of four waves per CU, four
    independent 32x32x16 products per wave in flight) and the shader clock it runs at, from the
    ratio of the shader-clock counter to the 100 MHz reference counter over each wave's loop:
    median of 5 timed batches of 10 launches after 200 ms of warm-up launches."""
    import ctypes
    import statistics
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_71_amd", "libexact_calib.so"))
    lib.calib_mfma.restype = ctypes.c_int
    lib.calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    ticks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream()

    def run():
        rc = lib.calib_mfma(blocks, iters, sink.data_ptr(), ticks.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"calib_mfma failed ({rc})")

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        run()
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 10)
    ms = sorted(times)[2]
    flops = blocks * 4 * iters * 4 * 32768
    t = ticks.view(blocks, 2).cpu().numpy()
    ghz = statistics.median((t[:, 0] / t[:, 1] * 0.1).tolist())
    print(json.dumps({"mfma_bf16_TFLOPs": flops / (ms * 1e-3) / 1e12, "ms": ms, "shader_clock_GHz": ghz,
                      "TFLOPs_at_clock": PEAK_BF16_TFLOPS * ghz / 2.4, "workgroups": blocks, "iters": iters}))


def tiny_f32(reps=200):
    """Only the tiny fp32 forward (B=1 H=1 N=256 d=64, non-causal; seed 1001): 0.3 s of warm-up
    calls, then `reps` timed calls; prints the mean ms per call.  For a profile of its kernel."""
    import numpy as np
    import torch
    from exact_io_aware_71_amd import binding as attn
    from synth import default_scale, make_prefill
    attn.load()
    tp = make_prefill(1, 1, 1, 256, 64, "f32", seed=1001)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(tp[x])).to("cuda:0") for x in ("q", "k", "v"))
    to = torch.empty_like(tq)
    tl = torch.empty((1, 1, 256), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def run():
        attn.attn_fwd(tq, tk, tv, False, default_scale(64), o=to, lse=tl)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"workload": "attn_fwd B=1 H=1 N=256 d=64 fp32 non-causal", "ms_per_call": ms,
                      "TFLOPs": flops_fwd(1, 1, 256, 64, False) / (ms * 1e-3) / 1e12, "calls": reps}))


def prefill_d64(reps=200):
    """Only the batched prefill (B=4, H=16, N=1024, d=64, causal, with LSE; seed 1002): 300 ms of
    warm-up calls, then `reps` timed calls; prints the mean ms.  For a profile of its kernel."""
    import numpy as np
    import torch
    from exact_io_aware_71_amd import binding as attn
    from synth import default_scale, make_prefill
    attn.load()
    dev = torch.device("cuda:0")
    bp = make_prefill(4, 16, 16, 1024, 64, "bf16", seed=1002)
    bq, bk, bv = (torch.from_numpy(np.ascontiguousarray(bp[x]).view(np.int16)).view(torch.bfloat16).to(dev)
                  for x in ("q", "k", "v"))
    bo = torch.empty_like(bq)
    blse = torch.empty((4, 16, 1024), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        attn.attn_fwd(bq, bk, bv, True, default_scale(64), o=bo, lse=blse)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"workload": "attn_fwd B=4 H=16 N=1024 d=64 causal with LSE", "ms": ms,
                      "TFLOPs": flops_fwd(4, 16, 1024, 64, True) / (ms * 1e-3) / 1e12, "calls": reps}))


def prefill_d64_sweep(reps=200):
    """The causal d=64 forward on one batch of 16 heads at N = 128 .. 1024 (2 to 16 key tiles on
    the longest walk, 16 to 128 workgroups, so at most one per CU) and on the batched prefill
    (B=4): 300 ms of warm-up calls per shape, then `reps` timed calls; prints the mean ms per
    shape (host-bound below about 10 us).  Under a kernel trace the grid sizes tell the shapes
    apart: the kernel durations give the per-launch fixed cost and the per-tile time of a
    workgroup alone on its CU."""
    import numpy as np
    import torch
    from exact_io_aware_71_amd import binding as attn
    from synth import default_scale, make_prefill
    attn.load()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    out = []
    for B, N in ((1, 128), (1, 256), (1, 512), (1, 1024), (4, 1024)):
        bp = make_prefill(B, 16, 16, N, 64, "bf16", seed=1100 + N + B)
        bq, bk, bv = (torch.from_numpy(np.ascontiguousarray(bp[x]).view(np.int16)).view(torch.bfloat16).to(dev)
                      for x in ("q", "k", "v"))
        bo = torch.empty_like(bq)
        blse = torch.empty((B, 16, N), dtype=torch.float32, device=dev)

        def run():
            attn.attn_fwd(bq, bk, bv, True, default_scale(64), o=bo, lse=blse)

        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append({"B": B, "H": 16, "N": N, "workgroups": B * 16 * ((N + 127) // 128),
                    "ms": e0.elapsed_time(e1) / reps})
    print(json.dumps({"workload": "attn_fwd d=64 causal with LSE, N sweep", "shapes": out, "calls": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary workloads (chunked prefill, packed, block-sparse, d=64, "
                         "variable-length decode) so that a profile holds the timed step only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device copies (reference for HBM byte counters)")
    ap.add_argument("--atomic-add", action="store_true",
                    help="only time fp32 atomic adds in 64 x 128 tiles (calibration)")
    ap.add_argument("--stream-read", action="store_true",
                    help="only time a streaming read of a 4 GiB buffer (HBM read ceiling of a plain kernel)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time a plain loop of dense bf16 MFMAs and read the shader clock it runs at")
    ap.add_argument("--tiny-f32", action="store_true",
                    help="only time the tiny fp32 forward (B=1 H=1 N=256 d=64), for a profile of its kernel")
    ap.add_argument("--prefill-d64", action="store_true",
                    help="only time the batched d=64 prefill (B=4 H=16 N=1024 causal), for a profile of its kernel")
    ap.add_argument("--prefill-d64-sweep", action="store_true",
                    help="only the causal d=64 forward at N = 128 .. 1024 (one batch of 16 heads) and the batched prefill")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.atomic_add:
        atomic_add()
        return
    if args.stream_read:
        stream_read()
        return
    if args.prefill_d64_sweep:
        prefill_d64_sweep()
        return
    if args.prefill_d64:
        prefill_d64()
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.tiny_f32:
        tiny_f32()
        return

    import numpy as np
    import torch
    from exact_io_aware_71_amd import binding as attn
    from synth import default_scale, make_decode, make_prefill, make_varlen

    attn.load()
    dev = torch.device("cuda:0")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    B, H, N, d = 2, 16, 4096, 128
    scale = default_scale(d)
    log("generating inputs")
    tr = make_prefill(B, H, H, N, d, "bf16", seed=1004, with_dout=True)
    q, k, v, do = (to_dev(tr[x]) for x in ("q", "k", "v", "dout"))
    del tr
    DB, DHq, DHkv, DL = 64, 32, 8, 8192
    dec = make_decode(DB, DHq, DHkv, DL, d, seed=1005)
    dq_, dk_, dv_ = (to_dev(dec[x]) for x in ("q", "k", "v"))
    del dec

    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_b = torch.empty(attn.attn_bwd_workspace_bytes(B, H, H, N, d), dtype=torch.uint8, device=dev)
    splits = attn.attn_decode_auto_splits(DB, DHq, DHkv, DL, d)
    ws_d = torch.empty(attn.attn_decode_workspace_bytes(DB, DHq, DHkv, DL, d, 0), dtype=torch.uint8, device=dev)
    dec_o = torch.empty_like(dq_)
    dec_lse = torch.empty((DB, DHq), dtype=torch.float32, device=dev)
    # Per-sequence cache lengths for the variable-length decode line: uniform in [L/2, L].
    vlens = np.random.default_rng(1006).integers(DL // 2, DL + 1, DB).astype(np.int32)
    vlens_dev = torch.from_numpy(vlens).to(dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        attn.attn_fwd(q, k, v, True, scale, o=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        attn.attn_bwd(q, k, v, o, lse, do, True, scale, dq=gq, dk=gk, dv=gv, workspace=ws_b)
        if ev is not None:
            ev[2].record(stream)
        attn.attn_decode(dq_, dk_, dv_, scale, num_splits=0, o=dec_o, lse=dec_lse, workspace=ws_d)
        if ev is not None:
            ev[3].record(stream)

    # The shader clock needs some 25 ms of load to settle after an idle gap (inputs are built on
    # the host with the GPU idle): run the step for 0.3 s before the W warm-up steps, so that a
    # small W does not leave the ramp inside the timed steps.
    log(f"settling 0.3 s, then warmup {args.warmup} steps")
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.3:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_fwd = [e[0].elapsed_time(e[1]) for e in evs]
    t_bwd = [e[1].elapsed_time(e[2]) for e in evs]
    t_dec = [e[2].elapsed_time(e[3]) for e in evs]
    t_step = [e[0].elapsed_time(e[3]) for e in evs]
    ms_fwd, ms_bwd, ms_dec = (float(np.mean(x)) for x in (t_fwd, t_bwd, t_dec))
    ms_step = float(np.mean(t_step))

    # Secondary lines (skipped with --no-extras, e.g. under a profiler): each timed on its own,
    # outside the timed step.
    extras = {}
    if not args.no_extras:
        def time_call(fn, reps=20, warm_ms=40.0):
            """Mean ms of one call over `reps` back-to-back calls, after about `warm_ms` of
            back-to-back warm-up calls: inputs are generated on the host with the GPU idle, and
            after such a gap the shader clock takes some 25 ms of load to settle."""
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            fn()
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            for _ in range(min(4000, int(warm_ms / max(ev[0].elapsed_time(ev[1]), 1e-3)) + 3)):
                fn()
            ev[0].record(stream)
            for _ in range(reps):
                fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) / reps

        # Variable-length decode, outside the timed step: same cache, lengths vlens.
        ms_vdec = time_call(lambda: attn.attn_decode_varlen(dq_, dk_, dv_, vlens_dev, scale, num_splits=0, o=dec_o,
                                                            lse=dec_lse, workspace=ws_d))
        vdec_bytes = int(vlens.sum()) * DHkv * d * 2 * 2 + 2 * DB * DHq * d * 2 + DB * DHq * 4

        # Secondary forward lines, outside the timed step, FLOPs = 4 d per (query, key) pair the
        # mask keeps.  Chunked prefill: a 1024-token chunk appended to 7168 cached tokens
        # (Nk = 8192, causal aligned at the bottom right), B=4, Hq=32, Hkv=8, d=128.

        log("chunked prefill and packed variable-length forward")
        CB, CHq, CHkv, CNq, CNk = 4, 32, 8, 1024, 8192
        ch = make_prefill(CB, CHq, CHkv, CNq, d, "bf16", seed=1007, L=CNk)
        cq, ck, cv = (to_dev(ch[x]) for x in ("q", "k", "v"))
        del ch
        co = torch.empty_like(cq)
        clse = torch.empty((CB, CHq, CNq), dtype=torch.float32, device=dev)
        ms_chunk = time_call(lambda: attn.attn_fwd_kv(cq, ck, cv, True, scale, o=co, lse=clse))
        chunk_pairs = CNq * (CNk - CNq) + CNq * (CNq + 1) // 2
        f_chunk = 4.0 * d * CB * CHq * chunk_pairs
        del cq, ck, cv, co, clse
        # Packed batch: 12 sequences, lengths uniform in [256, 4096] (seed 1008), H=16, d=128, causal.
        vl = np.random.default_rng(1008).integers(256, 4097, 12)
        VH = 16
        px = make_varlen(vl, vl, VH, VH, d, "bf16", seed=1009, with_dout=True)
        pq, pk, pv, pdo = (to_dev(px[x]) for x in ("q", "k", "v", "dout"))
        pcu = torch.from_numpy(px["cu_q"]).to(dev)
        del px
        po = torch.empty_like(pq)
        plse = torch.empty((VH, int(vl.sum())), dtype=torch.float32, device=dev)
        ms_varlen = time_call(lambda: attn.attn_fwd_varlen(pq, pk, pv, pcu, pcu, int(vl.max()), True, scale, o=po,
                                                          lse=plse))
        f_varlen = 4.0 * d * VH * float(sum(int(n) * (int(n) + 1) // 2 for n in vl))
        pg = [torch.empty_like(pq), torch.empty_like(pk), torch.empty_like(pv)]
        pws = torch.empty(attn.attn_bwd_varlen_workspace_bytes(len(vl), VH, int(vl.sum())), dtype=torch.uint8, device=dev)
        ms_varlen_bwd = time_call(lambda: attn.attn_bwd_varlen(pq, pk, pv, po, plse, pdo, pcu, pcu, int(vl.max()),
                                                              int(vl.max()), True, scale, dq=pg[0], dk=pg[1], dv=pg[2],
                                                              workspace=pws))
        del pq, pk, pv, po, plse, pdo, pg, pws
        # Block-sparse: B=1, H=32, N=16384, d=128, causal; query block i keeps key blocks i-7 .. i
        # and block 0 (128x128 blocks), i.e. a 1024-key window plus the first block.
        SH, SN = 32, 16384
        sp = make_prefill(1, SH, SH, SN, d, "bf16", seed=1010, with_dout=True)
        sq_, sk_, sv_, sdo = (to_dev(sp[x]) for x in ("q", "k", "v", "dout"))
        del sp
        nbk = SN // 128
        bi, bj = np.meshgrid(np.arange(nbk), np.arange(nbk), indexing="ij")
        smask = ((((bi - bj) >= 0) & ((bi - bj) < 8)) | (bj == 0)).astype(np.uint8)
        smask_dev = torch.from_numpy(smask).to(dev)
        so = torch.empty_like(sq_)
        slse = torch.empty((1, SH, SN), dtype=torch.float32, device=dev)
        ms_sparse = time_call(lambda: attn.attn_fwd_blocksparse(sq_, sk_, sv_, smask_dev, True, scale, o=so, lse=slse))
        # Kept (query, key) pairs: whole kept blocks below the diagonal, plus the causal half (with
        # the diagonal) of each diagonal block.
        off = int(np.sum(smask * (bi > bj)))
        sparse_pairs = off * 128 * 128 + nbk * 128 * 129 // 2
        f_sparse = 4.0 * d * SH * sparse_pairs
        sg = [torch.empty_like(sq_), torch.empty_like(sk_), torch.empty_like(sv_)]
        sws = torch.empty(attn.attn_bwd_workspace_bytes(1, SH, SH, SN, d), dtype=torch.uint8, device=dev)
        ms_sparse_bwd = time_call(lambda: attn.attn_bwd_blocksparse(sq_, sk_, sv_, so, slse, sdo, smask_dev, True, scale,
                                                                    dq=sg[0], dk=sg[1], dv=sg[2], workspace=sws))
        del sq_, sk_, sv_, sdo, so, slse, sg, sws

        # Grouped-query training step: B=1, Hq=32, Hkv=8 (4 query heads per KV head), N=4096,
        # d=128, causal (seed 1012); the backward sums dK and dV over each group's query heads.
        GHq, GHkv, GN = 32, 8, 4096
        gp = make_prefill(1, GHq, GHkv, GN, d, "bf16", seed=1012, with_dout=True)
        gq, gk, gv, gdo = (to_dev(gp[x]) for x in ("q", "k", "v", "dout"))
        del gp
        go = torch.empty_like(gq)
        glse = torch.empty((1, GHq, GN), dtype=torch.float32, device=dev)
        ms_gqa_fwd = time_call(lambda: attn.attn_fwd(gq, gk, gv, True, scale, o=go, lse=glse))
        gg = [torch.empty_like(gq), torch.empty_like(gk), torch.empty_like(gv)]
        gws = torch.empty(attn.attn_bwd_workspace_bytes(1, GHq, GHkv, GN, d), dtype=torch.uint8, device=dev)
        ms_gqa_bwd = time_call(lambda: attn.attn_bwd(gq, gk, gv, go, glse, gdo, True, scale, dq=gg[0], dk=gg[1],
                                                     dv=gg[2], workspace=gws))
        f_gqa = flops_fwd(1, GHq, GN, d, True)
        del gq, gk, gv, gdo, go, glse, gg, gws

        # Multi-token decode: 4 tokens per sequence on the decode cache (16 (token, head) rows per
        # KV head), causal, seed 1011 for the queries.
        MT = 4
        mq = torch.from_numpy(np.ascontiguousarray(make_prefill(DB, DHq, DHkv, MT, d, "bf16", seed=1011)["q"])
                              .view(np.int16)).view(torch.bfloat16).to(dev)
        mo = torch.empty_like(mq)
        mlse = torch.empty((DB, DHq, MT), dtype=torch.float32, device=dev)
        mws = torch.empty(attn.attn_decode_multi_workspace_bytes(DB, DHq, DHkv, MT, DL, d, 0), dtype=torch.uint8,
                          device=dev)
        ms_mdec = time_call(lambda: attn.attn_decode_multi(mq, dk_, dv_, scale, causal=True, o=mo, lse=mlse,
                                                           workspace=mws))
        mdec_bytes = 2 * DB * DHkv * DL * d * 2 + 2 * DB * DHq * MT * d * 2 + DB * DHq * MT * 4
        del mq, mo, mlse, mws
        # Batched prefill, d=64: B=4, H=16, N=1024, causal, with LSE (seed 1002).  Its
        # arithmetic intensity (N/4 = 254 FLOP per byte) is below the ridge point (2516.6 TFLOP/s
        # over 8000 GB/s = 315), so the roofline bound is the memory side: Q, K, V, O and LSE once.
        bp = make_prefill(4, 16, 16, 1024, 64, "bf16", seed=1002)
        bq, bk, bv = (to_dev(bp[x]) for x in ("q", "k", "v"))
        del bp
        bo = torch.empty_like(bq)
        blse = torch.empty((4, 16, 1024), dtype=torch.float32, device=dev)
        ms_pre64 = time_call(lambda: attn.attn_fwd(bq, bk, bv, True, default_scale(64), o=bo, lse=blse))
        f_pre64 = flops_fwd(4, 16, 1024, 64, True)
        b_pre64 = 4 * 4 * 16 * 1024 * 64 * 2 + 4 * 16 * 1024 * 4
        floor_pre64 = max(f_pre64 / (PEAK_BF16_TFLOPS * 1e12), b_pre64 / (PEAK_HBM_GBS * 1e9)) * 1e3
        del bq, bk, bv, bo, blse
        # Tiny fp32 forward: B=1, H=1, N=256, d=64, non-causal (seed 1001); latency-bound.
        tp = make_prefill(1, 1, 1, 256, 64, "f32", seed=1001)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(tp[x])).to(dev) for x in ("q", "k", "v"))
        ms_tiny = time_call(lambda: attn.attn_fwd(tq, tk, tv, False, default_scale(64)))
        f_tiny = flops_fwd(1, 1, 256, 64, False)
        del tp, tq, tk, tv
        # Long-prefill sweep: B=1, H=32, d=128, Q and K x2 (seed 1003), N = 4096, 8192, 16384,
        # causal and not.
        log("long-prefill sweep")
        sweep = []
        for LN in (4096, 8192, 16384):
            lp = make_prefill(1, 32, 32, LN, d, "bf16", seed=1003, qk_mult=2.0)
            lq, lk, lv = (to_dev(lp[x]) for x in ("q", "k", "v"))
            del lp
            lo = torch.empty_like(lq)
            llse = torch.empty((1, 32, LN), dtype=torch.float32, device=dev)
            for lc in (True, False):
                ms_l = time_call(lambda: attn.attn_fwd(lq, lk, lv, lc, scale, o=lo, lse=llse), reps=10)
                tf = flops_fwd(1, 32, LN, d, lc) / (ms_l * 1e-3) / 1e12
                sweep.append({"N": LN, "causal": lc, "ms": ms_l, "TFLOPs": tf, "frac": tf / PEAK_BF16_TFLOPS})
            del lq, lk, lv, lo, llse
        extras = {
            "decode_varlen": {"GBps": vdec_bytes / (ms_vdec * 1e-3) / 1e9, "ms": ms_vdec,
                              "lengths": "uniform in [L/2, L], seed 1006, mean %.0f" % float(vlens.mean())},
            "fwd_chunk": {"TFLOPs": f_chunk / (ms_chunk * 1e-3) / 1e12, "ms": ms_chunk,
                          "workload": "attn_fwd_kv B=4 Hq=32 Hkv=8 Nq=1024 Nk=8192 d=128 causal (bottom right)"},
            "fwd_blocksparse": {"TFLOPs": f_sparse / (ms_sparse * 1e-3) / 1e12, "ms": ms_sparse,
                                "bwd_TFLOPs": 2.5 * f_sparse / (ms_sparse_bwd * 1e-3) / 1e12, "bwd_ms": ms_sparse_bwd,
                                "workload": "attn_fwd_blocksparse B=1 H=32 N=16384 d=128 causal, 128x128 blocks: "
                                            "8-block band + first block (%.1f%% of causal pairs kept)"
                                            % (100.0 * sparse_pairs / (SN * (SN + 1) / 2))},
            "fwd_varlen": {"TFLOPs": f_varlen / (ms_varlen * 1e-3) / 1e12, "ms": ms_varlen,
                           "bwd_TFLOPs": 2.5 * f_varlen / (ms_varlen_bwd * 1e-3) / 1e12, "bwd_ms": ms_varlen_bwd,
                           "workload": "attn_fwd_varlen 12 packed sequences, lengths uniform in [256, 4096] "
                                       "(seed 1008, total %d), H=16 d=128 causal" % int(vl.sum())},
            "train_gqa": {"fwd_TFLOPs": f_gqa / (ms_gqa_fwd * 1e-3) / 1e12, "fwd_ms": ms_gqa_fwd,
                          "bwd_TFLOPs": 2.5 * f_gqa / (ms_gqa_bwd * 1e-3) / 1e12, "bwd_ms": ms_gqa_bwd,
                          "workload": "attn_fwd + attn_bwd B=1 Hq=32 Hkv=8 N=4096 d=128 causal"},
            "decode_multi": {"GBps": mdec_bytes / (ms_mdec * 1e-3) / 1e9, "ms": ms_mdec,
                         "workload": "attn_decode_multi B=64 Hq=32 Hkv=8 T=4 L=8192 d=128 causal"},
            "fwd_prefill_d64": {"TFLOPs": f_pre64 / (ms_pre64 * 1e-3) / 1e12, "ms": ms_pre64,
                                "workload": "attn_fwd B=4 H=16 N=1024 d=64 causal with LSE",
                                "roofline": {"bound": "hbm", "achieved": b_pre64 / (ms_pre64 * 1e-3) / 1e9,
                                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                             "frac": floor_pre64 / ms_pre64, "floor_ms": floor_pre64,
                                             "bytes": b_pre64,
                                             "traffic": load_traffic("fwd_ilv_kernel<64,4,64,true,false>",
                                                                     source_digest("fwd.hip", "common.h"))}},
            "fwd_tiny_f32": {"ms": ms_tiny, "TFLOPs": f_tiny / (ms_tiny * 1e-3) / 1e12,
                             "workload": "attn_fwd B=1 H=1 N=256 d=64 fp32 non-causal (latency-bound)"},
            "fwd_long_prefill": {"workload": "attn_fwd B=1 H=32 d=128, Q and K x2, with LSE", "lines": sweep},
        }
    f_fwd = flops_fwd(B, H, N, d, True)
    f_bwd = 2.5 * f_fwd
    tflops = (f_fwd + f_bwd) / ((ms_fwd + ms_bwd) * 1e-3) / 1e12
    dec_bytes = 2 * DB * DHkv * DL * d * 2 + 2 * DB * DHq * d * 2 + DB * DHq * 4
    dec_gbs = dec_bytes / (ms_dec * 1e-3) / 1e9

    log(f"timed {args.steps} steps: {wall:.3f} s")
    # Quick spot check of the timed outputs against the oracle (a few rows / one batch).
    import oracle
    from synth import make_prefill as mp
    tr = mp(B, H, H, N, d, "bf16", seed=1004)
    rows = np.array([0, 1, 1000, N - 1])
    o_ref, _ = oracle.forward_rows(tr["q"][:1, :2], tr["k"][:1, :2], tr["v"][:1, :2], scale, True, rows)
    spot = float(np.abs(o[:1, :2, rows].float().cpu().numpy() - o_ref).max())
    del tr

    fwd_digest = source_digest("fwd.hip", "common.h")
    bwd_digest = source_digest("bwd.hip", "common.h")
    dec_digest = source_digest("decode.hip", "common.h")
    roofline = {
        "kernel": "fwd_ilv_kernel (attn_fwd, causal, B*H=32, N=4096, d=128)",
        "bound": "mfma", "achieved": f_fwd / (ms_fwd * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
    }
    roofline["frac"] = roofline["achieved"] / roofline["peak"]
    roofline["traffic"] = load_traffic("fwd_ilv_kernel<128,8,64,true,false>", fwd_digest)
    bwd_traffic = [load_traffic(kn, bwd_digest) for kn in ("bwd_dq_kernel<128,true,false,false>",
                                                           "bwd_dq_kernel<128,true,false,true>",
                                                           "bwd_dkdv_lag_kernel<128,true,false>")]
    roofline_bwd = {
        "kernel": "bwd_dq_kernel (two launches) + bwd_dkdv_lag_kernel (attn_bwd, causal, B*H=32, N=4096, d=128)",
        "bound": "mfma", "achieved": f_bwd / (ms_bwd * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": f_bwd / (ms_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "traffic": None if None in bwd_traffic else sum(bwd_traffic),
    }
    roofline_decode = {
        "kernel": "decode_split_kernel + decode_merge_kernel (attn_decode, B=64, Hq=32, Hkv=8, L=8192, d=128)",
        "bound": "hbm", "achieved": dec_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": dec_gbs / PEAK_HBM_GBS,
        "traffic": load_traffic("decode_split_kernel<128,4,false>", dec_digest), "splits": splits,
    }

    result = {
        "metric": "attn fwd/bwd TFLOP/s (4N^2d, causal halved) bf16 N=4096 d=128; decode HBM GB/s",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "attention training step B=2 H=16 N=4096 d=128 causal (fwd+bwd) + GQA decode "
                               "B=64 Hq=32 Hkv=8 L=8192 d=128", "parallelism": "none (one GPU)"},
        "fwd_TFLOPs": f_fwd / (ms_fwd * 1e-3) / 1e12, "bwd_TFLOPs": f_bwd / (ms_bwd * 1e-3) / 1e12,
        "decode_GBps": dec_gbs,
        **extras,
        "ms": {"fwd": ms_fwd, "bwd": ms_bwd, "decode": ms_dec, "fwd_min": min(t_fwd), "bwd_min": min(t_bwd),
               "decode_min": min(t_dec), "wall_per_step": wall / args.steps * 1e3},
        "roofline": roofline, "roofline_bwd": roofline_bwd, "roofline_decode": roofline_decode,
        "spot_check_max_abs_err": spot,
        "gpu": torch.cuda.get_device_properties(0).gcnArchName,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
