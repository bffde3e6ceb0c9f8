"""Benchmark of block-causal ring-KV chunk attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1|...|7]

One step is one chunk of the chunk-wise autoregressive loop: for every denoise
step and every layer one bca_attend (the chunk's queries over the current
chunk plus the visible ring chunks), then one bca_append_chunk per layer that
writes the chunk's K/V into its ring slot. Each layer has its own cache, so
the K/V reads of a step come from HBM, not from the 256 MB Infinity Cache.

Workloads (synthetic inputs, random values of the stated shapes):
  1  WanToFight-shaped bf16: 12 heads, d 128, 1536 tokens per chunk, window of
     the current + previous 2 chunks (4608 keys), ring of 2 slots, 30 layers x
     4 denoise steps per chunk. The default and the reported line.
  2  Matrix-Game-4.0-shaped bf16: 24 heads, d 128, 405 tokens per chunk,
     reference chunk + last 20 chunks + current (8910 keys), 4 segments merged
     by log-sum-exp, 30 layers x 1 step.
  3  workload 1 streamed over 64 chunks (steps = 64): sustained time per chunk.
  4  workload 2 with an fp8-e4m3 K/V cache (per-head scales).
  5  workload 1 with rotary position embedding fused into the path: appends
     rotate K on the way into the ring (bca_append_chunk_rope) and attends
     rotate Q and the chunk's own K first (bca_attend_rope); base 10000,
     token r of chunk t at position t*n + r.
  6  training form of workload 1: a clip of 8 chunks (12 heads, d 128, 1536
     tokens each, window of the current + previous 2 chunks) attended at once
     with bca_attend_sequence, 30 layers per step, each with its own Q/K/V.
  7  workload 3 with the chunk step captured once in a HIP graph and replayed
     for every chunk (device-side chunk id read by the appends).
  8  workload 4 with one e4m3 scale per (layer, block, head), taken by each
     append from the chunk itself (only the appended block is re-quantised).

Prints one JSON line. `value` is algorithmic attention TFLOP/s over the whole
step (4*H*n*N_k*d per chunk-layer, appends included in the time), from a timed
region with no events inside the steps. `attend_us` and `roofline` come from
a second timed region of bca_attend calls only, back to back.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-causal attention TFLOP/s & µs per chunk-layer; % of MFMA peak"
# MI355X dense MFMA peak, published: bf16 for a bf16 cache; an fp8 cache
# contracts on the fp8 matrix cores, priced against the fp8 dense peak.
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "fp8_block": 5033.2,
               # Q K^T on the int8 matrix cores (5.0 POP/s dense), P V on fp8 (5.0)
               "int8k_block": 5033.2}
PEAK_HBM_GBS = 8000.0

CONFIGS = {
    1: dict(workload="wantofight_bf16_chunk", H=12, d=128, n=1536, S=2, W=2, R=0, G=0, L=30,
            steps_per_chunk=4, kv="bf16"),
    2: dict(workload="matrixgame4_bf16_chunk", H=24, d=128, n=405, S=20, W=20, R=1, G=4, L=30,
            steps_per_chunk=1, kv="bf16"),
    3: dict(workload="wantofight_bf16_stream64", H=12, d=128, n=1536, S=2, W=2, R=0, G=0, L=30,
            steps_per_chunk=4, kv="bf16"),
    4: dict(workload="matrixgame4_fp8cache_chunk", H=24, d=128, n=405, S=20, W=20, R=1, G=4,
            L=30, steps_per_chunk=1, kv="fp8"),
    5: dict(workload="wantofight_bf16_rope_chunk", H=12, d=128, n=1536, S=2, W=2, R=0, G=0,
            L=30, steps_per_chunk=4, kv="bf16", rope=10000.0),
    8: dict(workload="matrixgame4_fp8block_chunk", H=24, d=128, n=405, S=20, W=20, R=1, G=4,
            L=30, steps_per_chunk=1, kv="fp8_block"),
    7: dict(workload="wantofight_bf16_stream64_graph", H=12, d=128, n=1536, S=2, W=2, R=0, G=0,
            L=30, steps_per_chunk=4, kv="bf16", graph=True),
    9: dict(workload="matrixgame4_int8k_fp8v_block_chunk", H=24, d=128, n=405, S=20, W=20, R=1,
            G=4, L=30, steps_per_chunk=1, kv="int8k_block"),
    6: dict(workload="wantofight_bf16_sequence8", H=12, d=128, n=1536, C=8, W=2, P=0, G=0, L=30,
            kv="bf16", sequence=True),
}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def gen(shape, g, outliers=False):
    import torch
    z = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32)
    if outliers:
        u = torch.rand(shape, generator=g, device="cuda", dtype=torch.float32)
        z = torch.where(u < 0.01, 8.0 * torch.sign(z), z)
    return z.to(torch.bfloat16)


def cpu_baseline(cache, cfg, q0, k0, v0, t):
    """The oracle, untouched, on a bounded sample of the same workload: the
    chunk-layer of layer 0 restricted to the first few heads (heads are
    independent), scaled until the sample takes about 10 s of CPU work."""
    import numpy as np
    import torch

    import oracle

    H, d, n, W = cfg["H"], cfg["d"], cfg["n"], cfg["W"]
    K, V = cache.blocks(0)
    hist = {}
    for s in range(cfg["S"]):
        c = cache.slot_chunk(0, s)
        if c >= 0:
            hist[c] = (K[:, s].float().cpu().numpy(), V[:, s].float().cpu().numpy())
    ref = None
    if cfg["R"]:
        ref = (K[:, cfg["S"]].float().cpu().numpy(), V[:, cfg["S"]].float().cpu().numpy())
    if cfg["kv"] == "fp8":
        # the fp8 cache holds codes; the oracle attends over the dequantised values
        dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
        scale = 8.0 / 448.0
        hist = {c: (dec[K[:, s].cpu().numpy()] * scale, dec[V[:, s].cpu().numpy()] * scale)
                for c, s in ((c, c % cfg["S"]) for c in hist)}
        ref = (dec[K[:, cfg["S"]].cpu().numpy()] * scale, dec[V[:, cfg["S"]].cpu().numpy()] * scale)
    if cfg["kv"] in ("fp8_block", "int8k_block"):
        # codes with one scale per (block, head); int8 K codes on "int8k_block"
        dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
        KS, VS = (x.cpu().numpy() for x in cache.block_scales(0))
        deq = lambda codes, sc: dec[codes.cpu().numpy()] * sc[:, None, None]  # noqa: E731
        if cfg["kv"] == "int8k_block":
            deqk = lambda codes, sc: (codes.cpu().numpy().view(np.int8).astype(np.float64)  # noqa: E731
                                      * sc[:, None, None])
        else:
            deqk = deq
        hist = {c: (deqk(K[:, c % cfg["S"]], KS[c % cfg["S"]]),
                    deq(V[:, c % cfg["S"]], VS[c % cfg["S"]])) for c in hist}
        ref = (deqk(K[:, cfg["S"]], KS[cfg["S"]]), deq(V[:, cfg["S"]], VS[cfg["S"]]))
    qn, kn, vn = (x.float().cpu().numpy() for x in (q0, k0, v0))
    n_vis_blocks = 1 + sum(1 for c in hist if t - W <= c <= t - 1) + (1 if cfg["R"] else 0)
    nk = n_vis_blocks * n

    def run(hs):
        h_hist = {c: (kv[0][:hs].transpose(1, 0, 2), kv[1][:hs].transpose(1, 0, 2))
                  for c, kv in hist.items()}
        h_ref = None if ref is None else (ref[0][:hs].transpose(1, 0, 2),
                                          ref[1][:hs].transpose(1, 0, 2))
        t0 = time.perf_counter()
        oracle.attend(qn[:, :hs], kn[:, :hs], vn[:, :hs], h_hist, t=t, W=W,
                      scale=1 / math.sqrt(d), ref=h_ref, use_ref=bool(cfg["R"]))
        return time.perf_counter() - t0

    hs = 1
    dt = run(hs)
    if dt < 3.0 and H > 1:
        hs = min(H, max(2, int(math.ceil(10.0 / max(dt, 1e-3)))))
        dt = run(hs)
    # still short of ~10 s with every head: repeat the sample
    reps = 1
    if dt < 8.0:
        reps = max(1, int(math.ceil(10.0 / max(dt, 1e-3))))
        dt = dt + sum(run(hs) for _ in range(reps - 1))
    flops = 4.0 * hs * n * nk * d * reps
    v1, r1, d1 = cpu_baseline_one_core(run, lambda h: 4.0 * h * n * nk * d,
                                       dt / (hs * reps) * oracle.threads())
    model, nproc = host_cpu()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"layer 0 chunk-layer, {hs} of {H} heads x {n} query rows x {nk} keys, "
                      f"{reps} time(s) (fp64 dense-mask oracle, {dt:.1f} s in all)",
            "value_1core": v1,
            "sample_1core": (f"1 of {H} heads, {r1} time(s) on one thread ({d1:.1f} s)"
                             if v1 is not None else "left out: over 40 s on one thread"),
            "cpu_model": model, "nproc": nproc}


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo, what lscpu reports as Model
    name) and the number of cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return model, nproc


def cpu_baseline_one_core(run_sample, flops_of, est_s):
    """The same oracle sample on one thread: run_sample(hs) times the oracle
    on hs heads; repeated until about 5 s of CPU work. est_s estimates one
    head on one thread (from the threaded run); above 40 s the one-thread run
    is left out (None) so the benchmark stays within minutes."""
    import oracle
    if est_s > 40.0:
        return None, 0, 0.0
    before = oracle.threads()
    oracle.set_threads(1)
    try:
        dt, reps = run_sample(1), 1
        while dt < 5.0 and reps < 64:
            dt += run_sample(1)
            reps += 1
    finally:
        oracle.set_threads(before)
    return flops_of(1) * reps / dt / 1e12, reps, dt


_PEAK_MEASURED = {}


def measure_mfma_peak(kind="bf16"):
    """Dense MFMA rate measured on this GPU at the clock it runs at under load:
    the library's probe kernel issues 32x32 MFMAs back to back (bf16
    32x32x16, or e4m3 32x32x64 for kind "fp8") on every SIMD, one work group of
    8 waves per compute unit, timed with events on the stream it runs on; best
    of three launches after a first that loads the code."""
    if kind in _PEAK_MEASURED:
        return _PEAK_MEASURED[kind]
    import ctypes

    import torch

    import attention_bca_attend_amd as bca
    lib = bca.load_library()
    name = "bf16" if kind == "bf16" else "fp8"
    launch = getattr(lib, f"bca_probe_mfma_{name}")
    flops = getattr(lib, f"bca_probe_mfma_{name}_flops")
    launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    launch.restype = ctypes.c_int
    flops.argtypes = [ctypes.c_int, ctypes.c_int]
    flops.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty((cus * 8,), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    iters = 20000
    best = 0.0
    for rep in range(4):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = launch(cus, iters, ctypes.c_void_p(out.data_ptr()),
                    ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"MFMA probe launch failed ({rc})")
        torch.cuda.synchronize()
        if rep == 0:
            continue
        best = max(best, flops(cus, iters) / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    _PEAK_MEASURED[kind] = round(best, 1)
    return _PEAK_MEASURED[kind]


def roofline_mfma(achieved, kind, traffic, kernel):
    """The roofline object of an MFMA-bound kernel: the published dense peak of
    its operand type, and beside it the rate the probe measures on this GPU."""
    peak = PEAK_TFLOPS[kind]
    meas = measure_mfma_peak("bf16" if kind == "bf16" else "fp8")
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": kernel, "peak_measured": meas,
            "frac_measured": round(achieved / meas, 4) if meas > 0 else None}


def sequence_flops(H, d, n, C, W, P):
    """Algorithmic FLOP of one whole-sequence call: chunk c's n queries each
    meet P + (min(c, W) + 1) n keys, 4 d FLOP per (query, key) pair."""
    return sum(4.0 * H * n * (P + (min(c, W) + 1) * n) * d for c in range(C))


def cpu_baseline_sequence(cfg, q, k, v):
    """The oracle's whole-sequence form on layer 0, restricted to the first few
    heads (heads are independent), scaled until the sample takes about 10 s."""
    import oracle

    H, d, n, C, W, P = (cfg[x] for x in ("H", "d", "n", "C", "W", "P"))
    qn, kn, vn = (x.float().cpu().numpy() for x in (q, k, v))

    def run(hs):
        t0 = time.perf_counter()
        oracle.attend_sequence(qn[:, :hs], kn[:, :hs], vn[:, :hs], n, W, P, 1 / math.sqrt(d))
        return time.perf_counter() - t0

    hs = 1
    dt = run(hs)
    if dt < 3.0 and H > 1:
        hs = min(H, max(2, int(math.ceil(10.0 / max(dt, 1e-3)))))
        dt = run(hs)
    flops = sequence_flops(hs, d, n, C, W, P)
    v1, r1, d1 = cpu_baseline_one_core(run, lambda h: sequence_flops(h, d, n, C, W, P),
                                       dt / hs * oracle.threads())
    model, nproc = host_cpu()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"layer 0 whole sequence, {hs} of {H} heads x {C} chunks of {n} tokens "
                      f"(fp64 dense-mask oracle, {dt:.1f} s)",
            "value_1core": v1,
            "sample_1core": (f"1 of {H} heads, {r1} time(s) on one thread ({d1:.1f} s)"
                             if v1 is not None else "left out: over 40 s on one thread"),
            "cpu_model": model, "nproc": nproc}


def main_graph(args, cfg):
    """Workload 7: the chunk step (every attend, one device-id append per layer,
    the counter advance) captured once and replayed per chunk."""
    import torch

    import attention_bca_attend_amd as bca

    H, d, n, S, W, G, L = (cfg[k] for k in ("H", "d", "n", "S", "W", "G", "L"))
    spc = cfg["steps_per_chunk"]
    steps = args.steps if args.steps is not None else 64
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda")
    g.manual_seed(20261202)
    log(f"config {args.config}: {cfg}")
    cache = bca.Cache(L, H, d, n, S, kv_dtype="bf16")
    Q = [gen((n, H, d), g) for _ in range(L)]
    Kc = [gen((n, H, d), g) for _ in range(L)]
    Vc = [gen((n, H, d), g) for _ in range(L)]
    O = torch.empty((n, H, d), dtype=torch.bfloat16, device="cuda")
    LSE = torch.empty((H, n), dtype=torch.float32, device="cuda")
    for l in range(L):
        for c in range(S):
            cache.append_chunk(l, c, gen((n, H, d), g), gen((n, H, d), g))
    t_chunk = S
    spec = cache.spec(t_chunk, W, num_segments=G)
    ws = cache.workspace(spec)
    plan = cache.plan(0, spec)
    nk = plan["visible_keys"]
    flop_cl = 4.0 * H * n * nk * d
    for l in range(L):
        if not cache.replayable(l, spec):
            raise SystemExit("chunk step is not replayable for this workload")
    d_chunk = torch.full((1,), t_chunk, dtype=torch.int64, device="cuda")
    # one eager step first (loads the code objects, and it is chunk S)
    for _ in range(spc):
        for l in range(L):
            cache.attend(l, Q[l], Kc[l], Vc[l], spec, out=O, lse=LSE, workspace=ws)
    for l in range(L):
        cache.append_chunk_dev(l, d_chunk, Kc[l], Vc[l])
    bca.Cache.advance_counter(d_chunk)
    torch.cuda.synchronize()
    for l in range(L):
        cache.set_slot_chunk(l, t_chunk % S, t_chunk)
    t_chunk += 1
    spec = cache.spec(t_chunk, W, num_segments=G)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(spc):
            for l in range(L):
                cache.attend(l, Q[l], Kc[l], Vc[l], spec, out=O, lse=LSE, workspace=ws)
        for l in range(L):
            cache.append_chunk_dev(l, d_chunk, Kc[l], Vc[l])
        bca.Cache.advance_counter(d_chunk)
    torch.cuda.synchronize()

    def replay():
        nonlocal t_chunk
        graph.replay()
        for l in range(L):
            cache.set_slot_chunk(l, t_chunk % S, t_chunk)
        t_chunk += 1

    for _ in range(args.warmup):
        replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    per_chunk = []
    host_s = 0.0
    start.record()
    for _ in range(steps):
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        h0 = time.perf_counter()
        replay()
        host_s += time.perf_counter() - h0
        c1.record()
        per_chunk.append((c0, c1))
    end.record()
    torch.cuda.synchronize()
    assert int(d_chunk.item()) == t_chunk, "device chunk counter out of step"
    ms_step = start.elapsed_time(end) / steps
    chunk_ms = [a.elapsed_time(b) for a, b in per_chunk]
    n_attend = spc * L
    tflops = n_attend * flop_cl / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    log(f"{steps} replayed chunks: {ms_step:.3f} ms per chunk, {tflops:.1f} TFLOP/s")
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "heads": H, "head_dim": d, "chunk_tokens": n,
                   "visible_keys": nk, "ring_slots": S, "history": W, "reference": False,
                   "segments": G if G else "auto", "layers": L,
                   "denoise_steps_per_chunk": spc, "batch": 1, "graph": True},
        "us_per_chunk_layer": round(ms_step * 1e3 / n_attend, 3),
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "chunk_ms_min_max": [round(min(chunk_ms), 4), round(max(chunk_ms), 4)],
        "host_ms_per_step": round(host_s * 1e3 / steps, 4),
        "roofline": roofline_mfma(tflops, "bf16", measured_traffic(cfg["workload"]),
                                  "replayed chunk step (attends with appends, whole-step "
                                  "time)"),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(cache, dict(cfg, R=0), Q[0], Kc[0], Vc[0],
                                              t_chunk)
    print(json.dumps(result), flush=True)


def main_sequence(args, cfg):
    """Workload 6: one step = one whole-sequence call per layer."""
    import torch

    import attention_bca_attend_amd as bca

    H, d, n, C, W, P, G, L = (cfg[k] for k in ("H", "d", "n", "C", "W", "P", "G", "L"))
    steps = args.steps if args.steps is not None else 5
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda")
    g.manual_seed(20261202)
    log(f"config {args.config}: {cfg}")
    Q = [gen((C * n, H, d), g) for _ in range(L)]
    K = [gen((P + C * n, H, d), g) for _ in range(L)]
    V = [gen((P + C * n, H, d), g) for _ in range(L)]
    O = torch.empty((C * n, H, d), dtype=torch.bfloat16, device="cuda")
    spec = bca.bca_sequence_spec(H, d, n, C, P, W, G, 1.0 / math.sqrt(d))
    need = bca.bca_attend_sequence_workspace_bytes(spec, bca.BF16)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    LSE = torch.empty((C, H, n), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    flop_call = sequence_flops(H, d, n, C, W, P)

    def call(l):
        bca.bca_attend_sequence(spec, Q[l].data_ptr(), K[l].data_ptr(), V[l].data_ptr(),
                                bca.BF16, O.data_ptr(), LSE.data_ptr(), ws.data_ptr(), need,
                                stream)

    def run_step():
        for l in range(L):
            call(l)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    # one event pair around the K steps and one per step, none inside a step;
    # the step is nothing but the whole-sequence calls, so the same region
    # gives the per-call time
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    per_step = []
    start.record()
    for _ in range(steps):
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        run_step()
        c1.record()
        per_step.append((c0, c1))
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    step_ms = [a.elapsed_time(b) for a, b in per_step]
    call_us = ms_step * 1e3 / L
    tflops = L * flop_call / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    log(f"{steps} steps: {ms_step:.3f} ms/step, {call_us:.1f} us per sequence call, "
        f"{tflops:.1f} TFLOP/s")
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "heads": H, "head_dim": d, "chunk_tokens": n,
                   "chunks": C, "history": W, "prefix_tokens": P,
                   "segments": G if G else "auto", "layers": L, "batch": 1},
        "us_per_chunk_layer": round(call_us / C, 3),
        "sequence_call_us": round(call_us, 3),
        "pct_mfma_peak": round(100.0 * tflops / peak, 2),
        "step_ms_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
        "roofline": roofline_mfma(tflops, "bf16", measured_traffic(cfg["workload"]),
                                  f"bca_attend_sequence: {C} x (attn_bf16_kernel + "
                                  f"merge_lanes_kernel where split)"),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline_sequence(cfg, Q[0], K[0], V[0])
    print(json.dumps(result), flush=True)


KERNEL_SOURCE = os.path.join(ROOT, "attention_bca_attend_amd", "csrc", "bca_kernels.hip")
COPY_BYTES = 512 << 20


def kernel_source_sha256():
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the attention kernel for this workload, from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by what the same
    counters read for a copy of known size; None when there is no summary or
    the kernel source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return t.get("bytes_per_launch")


def copy_calibration():
    """A plain device copy of COPY_BYTES, three times: under rocprofv3 --pmc the
    copy kernel's FETCH_SIZE and WRITE_SIZE per dispatch are what the counters
    read for COPY_BYTES moved each way."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "dispatches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=1, choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the copy of known size that calibrates the traffic counters")
    ap.add_argument("--segments", type=int, default=None,
                    help="override the workload's segment count (0: the planner's own split)")
    ap.add_argument("--layers", type=int, default=None,
                    help="profiling runs only: fewer layers (each layer's launches are alike; "
                         "counter collection serialises every dispatch)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch

    import attention_bca_attend_amd as bca

    cfg = dict(CONFIGS[args.config])
    if args.layers:
        cfg["L"] = args.layers
    if args.segments is not None:
        cfg["G"] = args.segments
    if cfg.get("sequence"):
        main_sequence(args, cfg)
        return
    if cfg.get("graph"):
        main_graph(args, cfg)
        return
    steps = args.steps if args.steps is not None else (64 if args.config == 3 else 5)
    H, d, n, S, W, R, G, L = (cfg[k] for k in ("H", "d", "n", "S", "W", "R", "G", "L"))
    spc = cfg["steps_per_chunk"]
    fp8 = cfg["kv"] in ("fp8", "fp8_block", "int8k_block")
    rope_base = cfg.get("rope")
    rope = (lambda t: (rope_base, t * n)) if rope_base else (lambda t: None)
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda")
    g.manual_seed(20261202)

    log(f"config {args.config}: {cfg}")
    cache = bca.Cache(L, H, d, n, S, has_ref=bool(R), kv_dtype=cfg["kv"])
    if cfg["kv"] == "fp8":
        for l in range(L):
            cache.set_kv_scales(l, [8.0 / 448.0] * H, [8.0 / 448.0] * H)
    # per-layer Q/K/V of the current chunk, resident in HBM
    Q = [gen((n, H, d), g) for _ in range(L)]
    Kc = [gen((n, H, d), g, outliers=fp8) for _ in range(L)]
    Vc = [gen((n, H, d), g, outliers=fp8) for _ in range(L)]
    O = torch.empty((n, H, d), dtype=torch.bfloat16, device="cuda")
    LSE = torch.empty((H, n), dtype=torch.float32, device="cuda")
    # fill the ring (chunks 0..S-1) and the reference
    for l in range(L):
        if R:
            cache.append_chunk(l, 0, gen((n, H, d), g, fp8), gen((n, H, d), g, fp8), is_ref=True,
                               rope=rope(0))
        for c in range(S):
            cache.append_chunk(l, c, gen((n, H, d), g, fp8), gen((n, H, d), g, fp8),
                               rope=rope(c))
        if l % 10 == 9 or l == L - 1:
            torch.cuda.synchronize()
            log(f"set-up: ring of layers 0..{l} filled")
    torch.cuda.synchronize()
    t_chunk = S
    spec0 = cache.spec(t_chunk, W, use_ref=bool(R), num_segments=G)
    ws = cache.workspace(spec0, rope=rope_base is not None)
    plan = cache.plan(0, spec0)
    nk = plan["visible_keys"]
    flop_cl = 4.0 * H * n * nk * d
    log(f"plan: {plan['workgroups']} work groups, {plan['kv_tiles']} key tiles, "
        f"max segments {plan['max_pieces']}, merge {plan['merge']}, N_k {nk}")

    def run_chunk(t):
        spec = cache.spec(t, W, use_ref=bool(R), num_segments=G)
        for _ in range(spc):
            for l in range(L):
                cache.attend(l, Q[l], Kc[l], Vc[l], spec, out=O, lse=LSE, workspace=ws,
                             rope=rope(t))
        for l in range(L):
            cache.append_chunk(l, t, Kc[l], Vc[l], rope=rope(t))

    for _ in range(args.warmup):
        run_chunk(t_chunk)
        t_chunk += 1
    torch.cuda.synchronize()
    # timed region 1: K whole steps, one event pair per step and none inside
    # it (an event between kernels costs several microseconds of its own)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    per_chunk = []
    host_s = 0.0
    start.record()
    for i in range(steps):
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        h0 = time.perf_counter()
        run_chunk(t_chunk)
        host_s += time.perf_counter() - h0
        c1.record()
        per_chunk.append((c0, c1))
        t_chunk += 1
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / steps
    chunk_ms = [a.elapsed_time(b) for a, b in per_chunk]
    # timed region 2: the dominant launch alone. The attends of up to 5 steps
    # of the next chunk, back to back as in a step, between one event pair on
    # the stream they run on; the average is that region's time per call.
    spec = cache.spec(t_chunk, W, use_ref=bool(R), num_segments=G)
    a_steps = max(1, min(steps, 5))
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record()
    for _ in range(a_steps * spc):
        for l in range(L):
            cache.attend(l, Q[l], Kc[l], Vc[l], spec, out=O, lse=LSE, workspace=ws,
                         rope=rope(t_chunk))
    a1.record()
    torch.cuda.synchronize()
    attend_us = a0.elapsed_time(a1) / (a_steps * spc * L) * 1e3
    n_attend = spc * L
    flops_step = n_attend * flop_cl
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg["kv"]]
    achieved = flop_cl / (attend_us * 1e-6) / 1e12
    log(f"{steps} steps: {ms_step:.3f} ms/step, attend {attend_us:.2f} us, "
        f"{tflops:.1f} TFLOP/s over the step, {achieved:.1f} TFLOP/s per attend")

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16" if not fp8 else "bf16 q / fp8-e4m3 kv" if cfg["kv"] == "fp8"
                  else "bf16 q / fp8-e4m3 kv, scales per block" if cfg["kv"] == "fp8_block"
                  else "bf16 q (int8 x2 in QK) / int8 k / fp8-e4m3 v, scales per block"),
        "data": "synthetic",
        "config": {"workload": cfg["workload"], "heads": H, "head_dim": d, "chunk_tokens": n,
                   "visible_keys": nk, "ring_slots": S, "history": W, "reference": bool(R),
                   "segments": G if G else "auto", "layers": L,
                   "denoise_steps_per_chunk": spc, "batch": 1,
                   "rope_base": rope_base},
        "us_per_chunk_layer": round(ms_step * 1e3 / n_attend, 3),
        "attend_us": round(attend_us, 3),
        "pct_mfma_peak": round(100.0 * achieved / peak, 2),
        "chunk_ms_min_max": [round(min(chunk_ms), 4), round(max(chunk_ms), 4)],
        "host_ms_per_step": round(host_s * 1e3 / steps, 4),
        "roofline": roofline_mfma(
            achieved, cfg["kv"], measured_traffic(cfg["workload"]),
            ("bca_attend_rope: rope_stage_kernel + " if rope_base else "bca_attend: ")
            + ("attn_fp8_kernel + append_fp8_kernel (chunk copy)" if cfg["kv"] == "fp8"
               else "attn_fp8_kernel (block scales) + append_amax_kernel + "
                    "append_fp8_kernel (chunk copy)" if cfg["kv"] == "fp8_block"
               else "attn_fp8_kernel (int8 K, block scales) + append_amax_kernel + "
                    "append_fp8_kernel (chunk copy)" if fp8
               else "attn_bf16_kernel")
            + (" + merge_lanes_kernel" if plan["merge"] else "")),
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(cache, cfg, Q[0], Kc[0], Vc[0], t_chunk)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
