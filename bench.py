#!/usr/bin/env python3
"""Benchmark of the Parallax attention hot path on one MI355X (gfx950).

Default (--workload suite): the decode batch x ctx sweep the metric is quoted
over -- batch {1, 16, 128, 1024, 2048} x ctx {128, 1024, 8192, 32768}, 16 query
/ 8 KV heads, d = 128, contiguous bf16 KV cache, fp32 q / rho / out; points
whose cache exceeds 200 GB are skipped -- each point gated on parity with the
fp64 oracle (every sequence up to a 4 GiB cache, else eight sampled ones) and
timed beside that oracle.  The headline `value` / `ms_per_step` is the largest
single-GPU point, batch 1024 x 32768 tokens (a 137 GB cache); one step = one
parallax_decode call over the whole batch, timed exactly --steps times after
--warmup untimed steps.  The same line carries the other workloads as
sub-records: decode at batch 8 x 4096, paged decode (256 sequences, ctx
U[128, 32768], 16-token pages), causal prefill (batch 4 x 8192) and its
backward pass, and the q / rho projection at 32768 tokens, each
parity-gated and with its oracle baseline.

The KV cache is resident in HBM before timing starts.  To keep the 256 MB
last-level cache from serving it, caches below 1 GiB are cloned R times (R x
KV >= 1 GiB) and the copies rotated, step i using copy i % R.  Steps are timed
with HIP events recorded on the stream the kernels are launched on.

Prints ONE JSON line.  Single workloads (for profiling): --workload decode,
paged, prefill, prefill_bwd, lla (decode with local linear attention's solved
probe), qr_proj (q and rho projections), sweep, copy (a plain device copy used
to calibrate the HBM byte counters).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "Parallax decode KV GB/s (% of HBM peak) + tokens/s over batch×ctx sweep"
HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
# elementwise bound of the backward's gradients, max |g - r| / (1 + |r|):
# twice the worst ratio of a model of the forward's bf16 numerators and the
# backward's bf16 weights (tests/test_backward_tolerance.py)
TAU_BWD = 0.1
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Decode over a bf16 cache runs on bf16 matrix cores (q, rho and the softmax
# weights enter as two-term bf16 splits; sums accumulate in fp32).
DECODE_DTYPE = "bf16"
_COMMON = ["parallax_local_linear_decode_amd/csrc/kernels.hpp",
           "parallax_local_linear_decode_amd/csrc/api.hip"]
KERNEL_SOURCES = {  # what the kernels of a workload are built from
    "decode": ["parallax_local_linear_decode_amd/csrc/decode.hip",
               "parallax_local_linear_decode_amd/csrc/lla_row.hpp"] + _COMMON,
    "paged": ["parallax_local_linear_decode_amd/csrc/decode.hip",
              "parallax_local_linear_decode_amd/csrc/lla_row.hpp"] + _COMMON,
    "prefill": ["parallax_local_linear_decode_amd/csrc/prefill.hip"] + _COMMON,
    "prefill_bwd": ["parallax_local_linear_decode_amd/csrc/prefill_bwd.hip"] + _COMMON,
}
KERNEL_SOURCES["decode_headline"] = KERNEL_SOURCES["decode"]
KERNEL_SOURCES["qr_proj"] = ["parallax_local_linear_decode_amd/csrc/proj.hip"] + _COMMON


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha(workload):
    """Hash of what a workload's kernels are built from: their sources and
    the compiler flags they are built with."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from parallax_local_linear_decode_amd import build
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(workload, []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
        flags = build.flags_for(os.path.basename(rel))
        h.update(" ".join(f for f in flags if not f.startswith("-I")).encode())
    return h.hexdigest()[:16]


def traffic_for(workload):
    """HBM bytes per step (FETCH_SIZE + WRITE_SIZE of every kernel the step
    launches, calibrated against a plain copy) from committed counter runs,
    if they were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[workload]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha(workload):
        return None
    return float(t["bytes_per_launch"])


# ------------------------------------------------------------------ decode ---

def decode_bytes(B, Hq, Hkv, d, lens, kv_elem=2):
    """Algorithmic bytes: every K and V element once, plus q, rho and out."""
    return sum(lens) * Hkv * d * 2 * kv_elem + B * Hq * d * 4 * 3


# Least wall time of warm-up work before a timed region: an idle GPU needs
# on the order of 0.1 s of load to reach its working clock, and a short
# workload's W warm-up launches alone can end before that.
MIN_WARMUP_SECONDS = 0.25


def time_launches(torch, launch, n_bufs, steps, warmup):
    for i in range(warmup):
        launch(i % n_bufs)
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), warmup
    while warmup > 0 and time.perf_counter() - t0 < MIN_WARMUP_SECONDS:
        launch(i % n_bufs)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(i % n_bufs)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1000.0  # seconds


def single_call_us(torch, launch, n_bufs, calls=50):
    """Latency of one isolated call: events around it, the device idle
    before it (synchronised), cold input copy each time; median in us."""
    stream = torch.cuda.current_stream()
    ts = []
    for i in range(calls):
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        launch(i % n_bufs)
        end.record(stream)
        torch.cuda.synchronize()
        ts.append(start.elapsed_time(end) * 1e3)
    ts.sort()
    return round(ts[len(ts) // 2], 2)


def make_decode_launcher(torch, plx, sets, out, split, window=0):
    """Pre-marshalled C-ABI calls, one per input copy, so the host loop is a
    single ctypes call per step."""
    import ctypes
    lib = plx.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = []
    for inp in sets:
        a = plx._decode_args(inp.q, inp.rho, inp.k, inp.v, out, inp.scale, inp.seq_lens,
                             inp.block_table, None, split, window)
        n = ctypes.c_size_t(0)
        st = lib.parallax_decode_workspace_size(ctypes.byref(a), ctypes.byref(n))
        if st != 0:
            plx._raise(st, lib)
        ws = torch.zeros(max(n.value, 16), dtype=torch.uint8, device=out.device)
        calls.append((a, ws))

    def launch(i):
        a, ws = calls[i]
        st = lib.parallax_decode(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()),
                                 ws.numel(), stream)
        if st != 0:
            plx._raise(st, lib)
    return launch


def cpu_baseline_decode(inp, nbytes, budget_s=10.0, window=0):
    """The oracle (fp64 C, all host cores) on the same workload; repeated until
    about budget_s of wall time has passed."""
    import oracle
    from parallax_local_linear_decode_amd.workloads import host_array
    import numpy as np
    args = dict(q=host_array(inp.q), rho=host_array(inp.rho), k=host_array(inp.k),
                v=host_array(inp.v))
    sl = None if inp.seq_lens is None else host_array(inp.seq_lens).astype(np.int32)
    bt = None if inp.block_table is None else host_array(inp.block_table)
    threads = oracle.default_threads()
    reps, elapsed, ref = 0, 0.0, None
    while elapsed < budget_s and reps < 100000:
        t = time.perf_counter()
        ref = oracle.decode(args["q"], args["rho"], args["k"], args["v"], inp.scale,
                            seq_lens=sl, block_table=bt, window=window, threads=threads)
        elapsed += time.perf_counter() - t
        reps += 1
    per = elapsed / reps
    return ref, {"value": nbytes / per / 1e9, "unit": "GB/s", "cores": threads,
                 "kind": "oracle", "seconds_per_step": per,
                 "sample": f"the full workload, {reps} repetition(s), fp64 streaming form"}


def read_stream(torch, plx, nbytes, n_bufs, steps, warmup, decode_shape_wgs=0):
    """The HBM reference: a plain read-only streaming kernel (its own library,
    libparallax_probe.so) over the same bytes per step and the same number of
    rotating cold copies as the workload; GB/s."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(plx.__file__)), "libparallax_probe.so")
    if not os.path.exists(path):
        log(f"read stream: {path} missing (run the build); not reported")
        return None
    lib = ctypes.CDLL(path)
    lib.parallax_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.c_void_p]
    size = (nbytes + 15) // 16 * 16
    bufs = [torch.randint(0, 1 << 30, (size // 4,), dtype=torch.int32, device="cuda:0")
            for _ in range(n_bufs)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(i):
        if lib.parallax_probe_read(ctypes.c_void_p(bufs[i].data_ptr()), size,
                                   ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise SystemExit("read stream probe failed to launch")
    per = time_launches(torch, launch, n_bufs, steps, warmup) / steps
    rec = {"gbps": round(size / per / 1e9, 2), "bytes": size, "cold_copies": n_bufs,
           "kernel": "grid-stride 16-byte loads, 2048 x 256 threads (libparallax_probe)"}
    if decode_shape_wgs:
        # the same bytes read in the decode kernel's shape with no arithmetic:
        # the floor that grid shape leaves for a decode step
        lib.parallax_probe_read_decode_shape.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                                         ctypes.c_int, ctypes.c_void_p,
                                                         ctypes.c_void_p]

        def launch2(i):
            if lib.parallax_probe_read_decode_shape(ctypes.c_void_p(bufs[i].data_ptr()), size,
                                                    decode_shape_wgs,
                                                    ctypes.c_void_p(sink.data_ptr()),
                                                    stream) != 0:
                raise SystemExit("decode-shape read probe failed to launch")
        per2 = time_launches(torch, launch2, n_bufs, steps, warmup) / steps
        rec["decode_shape"] = {"gbps": round(size / per2 / 1e9, 2), "us": round(per2 * 1e6, 2),
                               "kernel": f"{decode_shape_wgs} workgroups x 8 waves, one 32-row "
                                         "step of K and of V in flight per wave, no arithmetic"}
    del bufs
    torch.cuda.empty_cache()
    return rec


def run_decode(args, torch, plx):
    from parallax_local_linear_decode_amd.workloads import decode_inputs
    B, Hq, Hkv, d, L, W = args.batch, 16, 8, 128, args.ctx, args.window
    Lw = min(L, W) if W > 0 else L  # tokens each row reads
    dev = torch.device("cuda:0")
    kv_bytes = B * Hkv * Lw * d * 2 * 2
    n_bufs = max(1, math.ceil(args.cold_bytes / kv_bytes))  # rotation over the bytes read
    sets = [decode_inputs(B, Hq, Hkv, d, L, seed=i, device=dev) for i in range(n_bufs)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    launch = make_decode_launcher(torch, plx, sets, out, args.split, W)
    nbytes = decode_bytes(B, Hq, Hkv, d, [Lw] * B)

    # parity gate on the data being timed (copy 0) before any number is reported
    launch(0)
    torch.cuda.synchronize()
    cpu, parity = None, None
    if args.cpu_baseline and kv_bytes <= FULL_PARITY_KV:
        gpu0 = out.double().cpu().numpy()
        ref, cpu = cpu_baseline_decode(sets[0], nbytes, budget_s=args.cpu_seconds, window=W)
        ratio, rms = gate(gpu0, ref, 2e-2, 1e-3)
        parity = {"sequences": "all", "max_err_ratio": ratio, "rel_rms": rms}
    elif args.cpu_baseline and W <= 0:  # a large cache: sampled sequences
        import numpy as np
        rng = np.random.default_rng(B + L)
        rows = sorted({0, B - 1, *(int(x) for x in rng.integers(0, B, SAMPLED_SEQUENCES - 2))})
        parity, cpu = decode_oracle_check(torch, sets[0], out, rows, args.cpu_seconds, nbytes)

    secs = time_launches(torch, launch, n_bufs, args.steps, args.warmup)
    per = secs / args.steps
    warm = time_launches(torch, launch, 1, args.steps, args.warmup) / args.steps
    single = single_call_us(torch, launch, n_bufs)
    gbps = nbytes / per / 1e9
    key = "decode" if (B, L) == (8, 4096) else "decode_headline" if (B, L) == (1024, 32768) else None
    traffic = traffic_for(key) if W <= 0 and key else None
    del sets, launch, out  # the read stream needs the memory of a large cache
    torch.cuda.empty_cache()
    wgs = 256 if (B, L, W, args.split) == (8, 4096, 0, 0) else 0  # the library's grid there
    stream_ref = read_stream(torch, plx, kv_bytes, n_bufs, args.steps, args.warmup, wgs)
    return {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s",
        "ms_per_step": per * 1e3, "dtype": DECODE_DTYPE,
        "config": {"workload": f"decode: batch {B}, 16 query / 8 KV heads, d 128, ctx {L}, "
                               "contiguous bf16 KV cache, fp32 q/rho/out"
                               + (f", local window {W} (bytes of the window)" if W > 0 else ""),
                   "batch": B, "ctx": L, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "kv_dtype": "bf16", "cold_copies": n_bufs,
                   "split_tokens": args.split, "window": W},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": B / per, "kv_tokens_per_s": B * Lw / per,
        "warm_cache_gbps": round(nbytes / warm / 1e9, 2),
        "single_call_us": single,
        "read_stream": stream_ref,
        "frac_of_read_stream": None if not stream_ref else round(gbps / stream_ref["gbps"], 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "parity": parity, "cpu_baseline": cpu,
    }


def run_lla(args, torch, plx):
    """Decode with LLA's solved probe: per step, `--lla-iters` conjugate-
    gradient sweeps plus the kbar sweep and the final Parallax sweep over the
    same cache -- the per-token solve the Parallax page contrasts with its one
    sweep.  Reports the KV bytes all sweeps stream per second, and the same
    cache's single-sweep Parallax decode time beside it."""
    import numpy as np
    import oracle
    from parallax_local_linear_decode_amd.workloads import decode_inputs, host_array
    B, Hq, Hkv, d, L = args.batch, 16, 8, 128, args.ctx
    lam, iters = args.lla_lambda, args.lla_iters
    dev = torch.device("cuda:0")
    kv_bytes = B * Hkv * L * d * 2 * 2
    n_bufs = max(1, math.ceil(args.cold_bytes / kv_bytes))
    sets = [decode_inputs(B, Hq, Hkv, d, L, seed=i, device=dev) for i in range(n_bufs)]
    outs = [plx.parallax_decode_lla(s.q, s.k, s.v, lam=lam, iterations=iters, scale=s.scale)
            for s in sets[:1]]
    torch.cuda.synchronize()
    out, rho, resid = outs[0]
    # parity of copy 0 against the oracle's direct solve (sequences 0 and B-1)
    idx = [0, B - 1]
    ref_out, ref_rho = oracle.lla_decode(host_array(sets[0].q[idx]), host_array(sets[0].k[idx]),
                                         host_array(sets[0].v[idx]), sets[0].scale, lam)
    gate(rho[idx].double().cpu().numpy(), ref_rho, 1e-3, 1e-3)
    gate(out[idx].double().cpu().numpy(), ref_out, 1e-3, 1e-3)
    cpu = None
    if args.cpu_baseline:
        hq, hk, hv = (host_array(t) for t in (sets[0].q, sets[0].k, sets[0].v))
        t0 = time.perf_counter()
        oracle.lla_decode(hq, hk, hv, sets[0].scale, lam)
        secs = time.perf_counter() - t0
        cpu = {"value": B / secs, "unit": "tokens/s", "cores": oracle.default_threads(),
               "kind": "oracle", "seconds_per_step": secs,
               "sample": "the full workload once: numpy fp64 direct solves of the probe, then the "
                         "C oracle's decode"}
    ws = torch.empty(1 << 26, dtype=torch.uint8, device=dev)
    res = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(3)]
    rsd = torch.empty((B, Hq), dtype=torch.float32, device=dev)

    def launch(i):
        s = sets[i]
        plx.parallax_decode_lla(s.q, s.k, s.v, lam=lam, iterations=iters, scale=s.scale,
                                out=res[0], rho_out=res[1], resid=rsd, workspace=ws)

    secs = time_launches(torch, launch, n_bufs, args.steps, args.warmup)
    per = secs / args.steps
    zero = torch.zeros((B, Hq, d), dtype=torch.float32, device=dev)
    single = time_launches(torch, lambda i: plx.parallax_decode(
        sets[i].q, zero, sets[i].k, sets[i].v, scale=sets[i].scale, out=res[2]),
        n_bufs, args.steps, args.warmup) / args.steps
    sweeps = iters + 2
    nbytes = sweeps * decode_bytes(B, Hq, Hkv, d, [L] * B)
    gbps = nbytes / per / 1e9
    # Sweeps after the first re-read the same cache, partly from the 256 MB
    # last-level cache, so bytes over all sweeps per second is not an HBM
    # rate (it can exceed 8 TB/s); the meaningful figures are the step time
    # and its ratio to one Parallax sweep.
    return {
        "metric": "LLA solved-probe decode tokens/s",
        "value": round(B / per, 1), "unit": "tokens/s", "ms_per_step": per * 1e3,
        "dtype": DECODE_DTYPE,
        "config": {"workload": f"LLA decode: batch {B}, 16 query / 8 KV heads, d 128, ctx {L}, "
                               f"bf16 KV cache, lambda {lam}, {iters} CG iterations "
                               f"({sweeps} sweeps per step)",
                   "batch": B, "ctx": L, "lambda": lam, "iterations": iters,
                   "sweeps_per_step": sweeps, "cold_copies": n_bufs},
        "tokens_per_s": B / per,
        "max_rel_residual": float(resid.max().item()),
        "parallax_ms_per_step": single * 1e3,
        "lla_over_parallax_time": round(per / single, 2),
        "sweep_bytes_per_s_gb": round(gbps, 2),
        "roofline": None,
        "cpu_baseline": cpu,
    }


def run_qr_proj(args, torch, plx):
    """q = W_Q x and rho = W_R x in one launch: at decode sizes (a few
    tokens) bound by streaming the two weight matrices from HBM (reported in
    GB/s against 8 TB/s); at prefill sizes by the matrix cores (TFLOP/s)."""
    import oracle
    from parallax_local_linear_decode_amd.workloads import host_array
    T, D, Hq, d = args.tokens, args.model_dim, 16, 128
    N = Hq * d
    dev = torch.device("cuda:0")
    out_dtype = torch.float32 if T <= 256 else torch.bfloat16
    w_bytes = 2 * N * D * 2
    n_bufs = max(1, math.ceil(args.cold_bytes / w_bytes))
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
    ws = [((torch.randn((N, D), generator=g, device=dev) / D ** 0.5).to(torch.bfloat16),
           (torch.randn((N, D), generator=g, device=dev) / D ** 0.5).to(torch.bfloat16))
          for _ in range(n_bufs)]
    q = torch.empty((T, Hq, d), dtype=out_dtype, device=dev)
    rho = torch.empty_like(q)
    plx.parallax_qr_projection(x, *ws[0], num_q_heads=Hq, out_dtype=out_dtype, q=q, rho=rho)
    torch.cuda.synchronize()
    rows = list(range(min(T, 64)))
    rq, rr = oracle.qr_projection(host_array(x[rows]), host_array(ws[0][0]), host_array(ws[0][1]))
    tau = 1e-5 if out_dtype == torch.float32 else 2.0 ** -8
    pq = gate(q[rows].reshape(len(rows), -1).double().cpu().numpy(), rq, tau, 1e-2)
    pr = gate(rho[rows].reshape(len(rows), -1).double().cpu().numpy(), rr, tau, 1e-2)
    parity = {"rows": f"the first {len(rows)} token rows, every feature",
              "q": {"max_err_ratio": pq[0], "rel_rms": pq[1]},
              "rho": {"max_err_ratio": pr[0], "rel_rms": pr[1]}}
    cpu = None
    if args.cpu_baseline:
        Ts = min(T, 1024)  # a bounded sample of token rows at prefill sizes
        hx, hq_, hr_ = host_array(x[:Ts]), host_array(ws[0][0]), host_array(ws[0][1])
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 2.0:
            oracle.qr_projection(hx, hq_, hr_)
            reps += 1
        per_cpu = (time.perf_counter() - t0) / reps
        cpu = {"value": 2 * Ts * 2 * N * D / per_cpu / 1e12, "unit": "TFLOP/s",
               "cores": oracle.default_threads(), "kind": "oracle",
               "seconds_per_step": per_cpu * T / Ts,
               "sample": (f"the full workload, {reps} repetition(s)" if Ts == T else
                          f"the first {Ts} of {T} token rows, {reps} repetition(s), scaled by "
                          f"{T / Ts:g} for seconds_per_step") + ", numpy fp64 matmul"}
    # pre-marshalled C-ABI calls: the host loop must not be the bottleneck
    import ctypes
    lib = plx.load_library()
    margs = []
    for w_q, w_r in ws:
        a = plx.ProjectionArgs()
        a.struct_size = ctypes.sizeof(plx.ProjectionArgs)
        a.tokens, a.model_dim, a.num_q_heads, a.head_dim = T, D, Hq, d
        a.out_dtype = plx.PARALLAX_F32 if out_dtype == torch.float32 else plx.PARALLAX_BF16
        a.x, a.x_stride_t = x.data_ptr(), x.stride(0)
        a.w_q, a.w_r, a.w_stride_n = w_q.data_ptr(), w_r.data_ptr(), w_q.stride(0)
        a.q, a.q_stride_t, a.q_stride_h = q.data_ptr(), q.stride(0), q.stride(1)
        a.rho, a.rho_stride_t, a.rho_stride_h = rho.data_ptr(), rho.stride(0), rho.stride(1)
        margs.append(a)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(i):
        st = lib.parallax_qr_projection(ctypes.byref(margs[i]), stream)
        if st != 0:
            plx._raise(st, lib)

    secs = time_launches(torch, launch, n_bufs, args.steps, args.warmup)
    per = secs / args.steps
    flops = 2 * T * 2 * N * D
    nbytes = w_bytes + T * D * 2 + 2 * T * N * (4 if out_dtype == torch.float32 else 2)
    gbps, tflops = nbytes / per / 1e9, flops / per / 1e12
    hbm = T <= 256
    roof = ({"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None} if hbm else
            {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
             # counters were taken at 32768 tokens, model dim 2048
             "traffic": traffic_for("qr_proj") if (T, D) == (32768, 2048) else None})
    return {
        "metric": "q and rho projection in one launch: " + ("weight GB/s" if hbm else "TFLOP/s"),
        "value": round(gbps, 2) if hbm else round(tflops, 1),
        "unit": "GB/s" if hbm else "TFLOP/s", "ms_per_step": per * 1e3, "dtype": "bf16",
        "config": {"workload": f"q = W_Q x, rho = W_R x: {T} tokens, model dim {D}, 16 heads x "
                               f"128, bf16 weights, {'fp32' if hbm else 'bf16'} out",
                   "tokens": T, "model_dim": D, "cold_copies": n_bufs},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": T / per,
        "roofline": roof, "parity": parity, "cpu_baseline": cpu,
    }


def run_paged(args, torch, plx):
    from parallax_local_linear_decode_amd.workloads import paged_inputs
    import numpy as np
    dev = torch.device("cuda:0")
    inp = paged_inputs(256, 16, 8, 128, seed=0, rho_zero_rows=32, device=dev)
    lens = inp.seq_lens.cpu().tolist()
    out = torch.empty((256, 16, 128), dtype=torch.float32, device=dev)
    launch = make_decode_launcher(torch, plx, [inp], out, args.split)
    nbytes = decode_bytes(256, 16, 8, 128, lens) + sum((L + 15) // 16 for L in lens) * 4
    launch(0)
    torch.cuda.synchronize()
    if not torch.isfinite(out).all():
        raise SystemExit("paged: non-finite output")
    # parity of the timed data on sampled sequences (the rho = 0 ones among
    # them, the longest and the shortest); the oracle's time on them, scaled
    # by their share of the cached tokens, is the CPU baseline
    import oracle
    rng = np.random.default_rng(0)
    pick = sorted(set([0, 1, 2, 31, int(np.argmax(lens)), int(np.argmin(lens))] +
                      [int(x) for x in rng.choice(np.arange(32, 256), 10, replace=False)]))
    q, rho, k, v, sl, table = _paged_subset(torch, inp, pick)
    threads = oracle.default_threads()
    reps, csecs, ref = 0, 0.0, None
    while reps < 1 or (csecs < args.cpu_seconds and reps < 1000):
        t0 = time.perf_counter()
        ref = oracle.decode(q, rho, k, v, inp.scale, seq_lens=sl, block_table=table,
                            threads=threads)
        csecs += time.perf_counter() - t0
        reps += 1
    ratio, rms = gate(out[pick].double().cpu().numpy(), ref, 2e-2, 1e-3)
    share = sum(lens[i] for i in pick) / sum(lens)
    full = csecs / reps / share
    cpu = {"value": nbytes / full / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seconds_per_step": full, "extrapolated": True,
           "sample": f"{len(pick)} of 256 sequences ({100 * share:.1f}% of the cached tokens), "
                     f"{reps} repetition(s), fp64 streaming form; time scaled by cached tokens"}
    secs = time_launches(torch, launch, 1, args.steps, args.warmup)
    per = secs / args.steps
    gbps = nbytes / per / 1e9
    del inp, launch
    torch.cuda.empty_cache()
    stream_ref = read_stream(torch, plx, nbytes, 1, min(args.steps, 50), 3)
    return {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "ms_per_step": per * 1e3,
        "dtype": DECODE_DTYPE,
        "config": {"workload": "paged decode: batch 256, 16 query / 8 KV heads, d 128, "
                               "ctx U[128, 32768], 16-token pages, shuffled block table, bf16",
                   "batch": 256, "total_tokens": int(sum(lens)), "kv_gb": nbytes / 1e9},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "tokens_per_s": 256 / per, "kv_tokens_per_s": sum(lens) / per,
        "read_stream": stream_ref,
        "frac_of_read_stream": None if not stream_ref else round(gbps / stream_ref["gbps"], 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for("paged")},
        "parity": {"sequences": pick, "max_err_ratio": ratio, "rel_rms": rms},
        "cpu_baseline": cpu,
    }


def _paged_subset(torch, inp, batch_ids):
    """Host copies of the paged inputs of sequences `batch_ids`: a compact
    pool of their pages and a renumbered block table."""
    import numpy as np
    from parallax_local_linear_decode_amd.workloads import host_array
    table = inp.block_table.cpu()
    lens = inp.seq_lens.cpu()
    P = inp.k.shape[2]
    pages = [table[b, :(int(lens[b]) + P - 1) // P].long() for b in batch_ids]
    ids = torch.cat(pages).to(inp.k.device)
    new_table = np.zeros((len(batch_ids), max(len(x) for x in pages)), dtype=np.int32)
    off = 0
    for i, pg in enumerate(pages):
        new_table[i, :len(pg)] = np.arange(off, off + len(pg), dtype=np.int32)
        off += len(pg)
    sel = torch.as_tensor(batch_ids, dtype=torch.long, device=inp.q.device)
    return (host_array(inp.q[sel]), host_array(inp.rho[sel]), host_array(inp.k[ids]),
            host_array(inp.v[ids]), lens[list(batch_ids)].numpy().astype(np.int32), new_table)


SWEEP_BATCHES = (1, 16, 128, 1024, 2048)
SWEEP_CTX = (128, 1024, 8192, 32768)
SWEEP_MAX_KV = 200e9          # points with a larger cache are skipped
HEADLINE_POINT = (1024, 32768)  # the largest single-GPU point of the sweep
FULL_PARITY_KV = 4 << 30      # up to this cache size every sequence is checked
SAMPLED_SEQUENCES = 8


def clone_inputs(inp):
    """The same inputs in fresh device memory (a cold copy for the rotation)."""
    return dataclasses.replace(inp, q=inp.q.clone(), rho=inp.rho.clone(), k=inp.k.clone(),
                               v=inp.v.clone())


def decode_oracle_check(torch, inp, out, rows, cpu_seconds, nbytes):
    """Parity gate of decode outputs `out` on sequences `rows` against the
    oracle, which is timed on those sequences (repeated for about
    `cpu_seconds`) and scaled to the whole batch by its share of the cached
    tokens.  Returns (parity record, cpu_baseline record)."""
    import numpy as np
    import oracle
    from parallax_local_linear_decode_amd.workloads import host_array
    B = inp.q.shape[0]
    sel = torch.as_tensor(rows, dtype=torch.long, device=inp.q.device)
    hq, hr, hk, hv = (host_array(t[sel]) for t in (inp.q, inp.rho, inp.k, inp.v))
    threads = oracle.default_threads()
    reps, secs, ref = 0, 0.0, None
    while reps < 1 or (secs < cpu_seconds and reps < 100000):
        t0 = time.perf_counter()
        ref = oracle.decode(hq, hr, hk, hv, inp.scale, threads=threads)
        secs += time.perf_counter() - t0
        reps += 1
    ratio, rms = gate(out[sel].double().cpu().numpy(), ref, 2e-2, 1e-3)
    full = secs / reps * B / len(rows)  # every sequence has the same length
    every = len(rows) == B
    parity = {"sequences": "all" if every else rows, "max_err_ratio": ratio, "rel_rms": rms,
              "bound": "max |g-r|/(1+|r|) <= 2e-2 and rel-RMS <= 1e-3"}
    cpu = {"value": nbytes / full / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seconds_per_step": full, "extrapolated": not every,
           "sample": (f"{'all' if every else len(rows)} of {B} sequences, {reps} repetition(s) "
                      f"({secs:.2f} s), fp64 streaming form"
                      + ("" if every else "; time scaled by cached tokens to the whole batch"))}
    return parity, cpu


def decode_point(args, torch, plx, B, L, seed, steps=None, warmup=None, cpu_seconds=0.3):
    """One point of the sweep: seeded inputs, rotated cold copies, a parity
    gate and oracle baseline, then `steps` timed steps after `warmup` (by
    default enough steps for about 0.1 s of GPU time, at least --steps)."""
    import numpy as np
    from parallax_local_linear_decode_amd.workloads import decode_inputs
    Hq, Hkv, d = 16, 8, 128
    dev = torch.device("cuda:0")
    kv = B * Hkv * L * d * 2 * 2
    nbytes = decode_bytes(B, Hq, Hkv, d, [L] * B)
    n_bufs = max(1, math.ceil(args.cold_bytes / kv))
    inp = decode_inputs(B, Hq, Hkv, d, L, seed=seed, device=dev)
    sets = [inp] + [clone_inputs(inp) for _ in range(n_bufs - 1)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    launch = make_decode_launcher(torch, plx, sets, out, 0)
    launch(0)
    torch.cuda.synchronize()
    if kv <= FULL_PARITY_KV:
        rows = list(range(B))
    else:
        rng = np.random.default_rng(seed)
        rows = sorted({0, B - 1, *(int(x) for x in rng.integers(0, B, SAMPLED_SEQUENCES - 2))})
    parity, cpu = decode_oracle_check(torch, inp, out, rows, cpu_seconds, nbytes)
    if steps is None:  # about 0.1 s of timed GPU work, at least --steps
        est = time_launches(torch, launch, n_bufs, 3, 1) / 3
        steps = max(args.steps, min(20000, int(0.1 / max(est, 1e-7))))
        warmup = max(args.warmup, 3)
    per = time_launches(torch, launch, n_bufs, steps, warmup) / steps
    gbps = nbytes / per / 1e9
    rec = {"batch": B, "ctx": L, "kv_bytes": kv, "bytes_per_step": nbytes, "steps": steps,
           "cold_copies": n_bufs, "us_per_step": per * 1e6, "gbps": round(gbps, 2),
           "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2), "tokens_per_s": B / per,
           "kv_tokens_per_s": B * L / per,
           "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)},
           "parity": parity, "cpu_baseline": cpu}
    del sets, inp, out, launch
    torch.cuda.empty_cache()
    return rec


def sweep_points(args, torch, plx, headline=None):
    """Every point of the batch x ctx grid, in grid order; the `headline`
    point is timed with exactly --steps steps after --warmup."""
    points = []
    for i, (B, L) in enumerate((B, L) for B in SWEEP_BATCHES for L in SWEEP_CTX):
        kv = B * 8 * L * 128 * 2 * 2
        if kv > SWEEP_MAX_KV:
            points.append({"batch": B, "ctx": L, "kv_bytes": kv,
                           "skipped": "KV cache above 200 GB"})
            continue
        if kv * 1.05 + (1 << 30) > torch.cuda.mem_get_info()[0]:
            points.append({"batch": B, "ctx": L, "kv_bytes": kv, "skipped": "free HBM"})
            continue
        is_head = (B, L) == headline
        rec = decode_point(args, torch, plx, B, L, seed=1000 + i,
                           steps=args.steps if is_head else None,
                           warmup=args.warmup if is_head else None,
                           cpu_seconds=args.cpu_seconds if is_head else 0.3)
        log(json.dumps({k: rec[k] for k in ("batch", "ctx", "us_per_step", "gbps",
                                            "pct_hbm_peak")}))
        points.append(rec)
    return points


def run_sweep(args, torch, plx):
    points = sweep_points(args, torch, plx)
    return {"metric": METRIC, "value": None, "unit": "GB/s", "ms_per_step": None,
            "dtype": DECODE_DTYPE, "config": {"workload": "decode sweep: batch x ctx grid, "
                                                        "16/8 heads, d 128, bf16 KV"},
            "sweep": points, "roofline": None, "cpu_baseline": None}


def sweep_summary(points):
    """Per-point GB/s and fraction of the 8 TB/s peak at a glance, and the
    range over the points with ctx >= 4096."""
    ok = [p for p in points if "gbps" in p]
    long_ctx = [p["roofline"]["frac"] for p in ok if p["ctx"] >= 4096]
    return {"points_measured": len(ok), "points_skipped": len(points) - len(ok),
            "frac_hbm_ctx_ge_4096": {"min": min(long_ctx), "median": sorted(long_ctx)[len(long_ctx) // 2],
                                     "max": max(long_ctx)} if long_ctx else None,
            "table": [f"{p['batch']}x{p['ctx']}: {p['us_per_step']:.1f} us, {p['gbps']:.0f} GB/s, "
                      f"{p['pct_hbm_peak']:.1f}%" for p in ok]}


def run_suite(args, torch, plx):
    """The metric as quoted: the whole sweep, headlined by its largest
    single-GPU point, with the other workloads as sub-records."""
    points = sweep_points(args, torch, plx, headline=HEADLINE_POINT)
    head = next((p for p in points if (p["batch"], p["ctx"]) == HEADLINE_POINT and "gbps" in p),
                None)
    if head is None:
        raise SystemExit("the headline point (batch 1024 x 32768) could not be measured")
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup = max(args.steps, 200), max(args.warmup, 20)
    sub.cpu_seconds = 3.0
    recs = {}
    sub.batch, sub.ctx, sub.window, sub.split = 8, 4096, 0, 0
    recs["decode_b8_ctx4096"] = run_decode(sub, torch, plx)
    sub.ctx, sub.window = 32768, 4096  # the local window: each row's last 4096 tokens
    recs["decode_window4096"] = run_decode(sub, torch, plx)
    sub.ctx, sub.window = 4096, 0
    recs["lla"] = run_lla(sub, torch, plx)
    recs["paged"] = run_paged(sub, torch, plx)
    sub.head_dim, sub.q_heads, sub.kv_heads = 128, 16, 8
    sub.steps, sub.warmup = max(args.steps, 20), max(args.warmup, 3)
    recs["prefill"] = run_prefill(sub, torch, plx)
    sub.window = 1024
    recs["prefill_window1024"] = run_prefill(sub, torch, plx)
    sub.window = 0
    recs["prefill_bwd"] = run_prefill_bwd(sub, torch, plx)
    sub.tokens, sub.model_dim = 32768, 2048
    recs["qr_proj"] = run_qr_proj(sub, torch, plx)
    try:  # a context measurement: its failure must not cost the line
        probe = issue_probe(torch, plx)
    except (SystemExit, RuntimeError) as e:
        log(f"issue probe not reported: {e}")
        probe = None
    for r in recs.values():  # the sub-records' own JSON keys, minus the shared ones
        for k in ("metric", "dtype"):
            r.pop(k, None)
    B, L = HEADLINE_POINT
    per = head["us_per_step"] * 1e-6
    roof = dict(head["roofline"])
    roof["traffic"] = traffic_for("decode_headline")
    return {
        "metric": METRIC, "value": head["gbps"], "unit": "GB/s", "ms_per_step": per * 1e3,
        "dtype": DECODE_DTYPE,
        "config": {"workload": f"decode: batch {B}, 16 query / 8 KV heads, d 128, ctx {L}, "
                               "contiguous bf16 KV cache (137 GB), fp32 q/rho/out: the largest "
                               "single-GPU point of the batch x ctx sweep",
                   "batch": B, "ctx": L, "num_q_heads": 16, "num_kv_heads": 8, "head_dim": 128,
                   "kv_dtype": "bf16", "cold_copies": head["cold_copies"]},
        "pct_hbm_peak": head["pct_hbm_peak"], "tokens_per_s": head["tokens_per_s"],
        "kv_tokens_per_s": head["kv_tokens_per_s"], "parity": head["parity"],
        "roofline": roof, "cpu_baseline": head["cpu_baseline"],
        "sweep_summary": sweep_summary(points), "sweep": points, **recs,
        "issue_probe": probe, "host": host_info(),
    }


def issue_probe(torch, plx, steps=5, warmup=2):
    """How matrix-core and vector work share a SIMD (libparallax_probe): one
    workgroup of eight waves per CU, waves 0-3 running independent 16x16x32
    bf16 MFMAs and waves 4-7 (one beside each) independent fp32 FMAs or
    base-2 exponentials, each group alone and both together, and FMAs on two
    waves per SIMD (how much of the vector rate one wave issues).  `overlap` is
    (t_a + t_b - t_ab) / min(t_a, t_b): 1 when the two kinds of work run side
    by side, 0 when they take turns."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(plx.__file__)), "libparallax_probe.so")
    if not os.path.exists(path):
        log(f"issue probe: {path} missing (run the build); not reported")
        return None
    lib = ctypes.CDLL(path)
    lib.parallax_probe_issue.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(512, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    M, F, E = 40000, 160000, 40000  # iterations: about 2 ms alone each

    def timed(mode, valu_iters):
        def launch(i):
            if lib.parallax_probe_issue(mode, M, valu_iters, cus, ctypes.c_void_p(sink.data_ptr()),
                                        stream) != 0:
                raise SystemExit("issue probe failed to launch")
        return time_launches(torch, launch, 1, steps, warmup) / steps

    t_m, t_f, t_mf, t_ff = timed(1, F), timed(2, F), timed(3, F), timed(10, F)
    t_e, t_me = timed(6, E), timed(7, E)
    mfma_flops = cus * 4 * M * 8 * 16 * 16 * 32 * 2
    fma_flops = cus * 4 * 64 * F * 8 * 2

    def overlap(a, b, ab):
        return round((a + b - ab) / min(a, b), 3)
    return {
        "kernel": f"{cus} workgroups x 8 waves (one per CU); per SIMD one MFMA wave and one "
                  "vector wave, 8 independent chains each",
        "mfma_alone_us": round(t_m * 1e6, 1),
        "mfma_alone_tflops": round(mfma_flops / t_m / 1e12, 1),
        "fma_alone_us": round(t_f * 1e6, 1),
        "fma_alone_tflops": round(fma_flops / t_f / 1e12, 1),
        "fma_two_waves_per_simd_tflops": round(2 * fma_flops / t_ff / 1e12, 1),
        "mfma_with_fma_us": round(t_mf * 1e6, 1),
        "overlap_mfma_fma": overlap(t_m, t_f, t_mf),
        "exp_alone_us": round(t_e * 1e6, 1),
        "exp_alone_per_s": round(cus * 4 * 64 * E * 8 / t_e, 1),
        "mfma_with_exp_us": round(t_me * 1e6, 1),
        "overlap_mfma_exp": overlap(t_m, t_e, t_me),
    }


def run_issue(args, torch, plx):
    rec = issue_probe(torch, plx, args.steps, args.warmup)
    if rec is None:
        raise SystemExit("issue probe library missing")
    return {"metric": "MFMA and vector work on one SIMD (overlap)", "value": rec["overlap_mfma_fma"],
            "unit": "fraction", "ms_per_step": rec["mfma_with_fma_us"] * 1e-3, "dtype": "bf16",
            "config": {"workload": "issue probe: MFMA waves beside FMA or exp waves"},
            "roofline": None, "cpu_baseline": None, **rec}


def run_sdpa(args, torch, plx):
    """Context, not the method: torch's fused softmax attention (its flash
    backend on this ROCm build) on the decode and prefill shapes above,
    with equal head counts (the fused kernels take no grouped heads). The
    decode case streams the same 134 MB cache as batch 8 x 4096 at 16/8
    heads; the prefill case does the causal softmax-attention half of the
    Parallax prefill's matrix products (2 of 4)."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    F = torch.nn.functional
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(0)

    def rnd(*shape):
        return torch.randn(*shape, device=dev, dtype=torch.bfloat16, generator=gen)

    def timed(sets, causal):
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            def launch(i):
                F.scaled_dot_product_attention(*sets[i], is_causal=causal)
            launch(0)
            torch.cuda.synchronize()
            return time_launches(torch, launch, len(sets), args.steps, args.warmup) / args.steps
    B, H, L, d = 8, 8, 4096, 128
    sets = [(rnd(B, H, 1, d), rnd(B, H, L, d), rnd(B, H, L, d)) for _ in range(8)]
    t_dec = timed(sets, False)
    kv = B * H * L * d * 2 * 2
    del sets
    S, Hq = 8192, 16
    t_pf = timed([(rnd(4, Hq, S, d), rnd(4, Hq, S, d), rnd(4, Hq, S, d))], True)
    fl = 2 * 2 * d * causal_pairs(S) * 4 * Hq
    return {"metric": "torch fused softmax attention (flash backend), for context",
            "value": round(fl / t_pf / 1e12, 1), "unit": "TFLOP/s", "ms_per_step": t_pf * 1e3,
            "dtype": "bf16",
            "config": {"workload": "torch SDPA: decode 8 x 4096 at 8/8 heads; causal prefill "
                                   "4 x 8192 at 16/16 heads, d 128"},
            "roofline": None, "cpu_baseline": None,
            "decode_us": round(t_dec * 1e6, 2), "decode_gbps": round(kv / t_dec / 1e9, 1),
            "prefill_ms": round(t_pf * 1e3, 4), "prefill_tflops": round(fl / t_pf / 1e12, 1)}


def run_copy(args, torch, plx):
    """A plain device-to-device copy of a known size, to calibrate counters."""
    n = args.copy_bytes
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    secs = time_launches(torch, lambda i: b.copy_(a), 1, args.steps, args.warmup)
    per = secs / args.steps
    return {"metric": "device copy GB/s (read + write)", "value": 2 * n / per / 1e9,
            "unit": "GB/s", "ms_per_step": per * 1e3, "dtype": "u8",
            "config": {"workload": f"copy {n} bytes"}, "roofline": None, "cpu_baseline": None}


def causal_pairs(S, window=0):
    """(query, key) pairs of one causal sequence: row i sees i+1 keys, or
    min(i+1, window) with a local window."""
    if window <= 0 or window >= S:
        return S * (S + 1) // 2
    return window * (window + 1) // 2 + (S - window) * window


def prefill_flops(B, S, Hq, d, window=0):
    """Algorithmic flops: per causal (query, key) pair and query head, the two
    score products (q.k, rho.k) and the two value products (E v, E t v), each
    2*d flops."""
    return 4 * 2 * d * causal_pairs(S, window) * B * Hq


def run_prefill(args, torch, plx):
    import numpy as np
    import oracle
    from parallax_local_linear_decode_amd.workloads import host_array, prefill_inputs
    B, S, Hq, Hkv, d = 4, 8192, args.q_heads, args.kv_heads, args.head_dim
    dev = torch.device("cuda:0")
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, d, seed=0, device=dev)
    out = torch.empty((B, S, Hq, d), dtype=torch.float32, device=dev)
    import ctypes
    lib = plx.load_library()
    a = plx.PrefillArgs()
    a.struct_size = ctypes.sizeof(plx.PrefillArgs)
    a.batch, a.seq_len, a.num_q_heads, a.num_kv_heads, a.head_dim = B, S, Hq, Hkv, d
    a.scale, a.causal = scale, 1
    a.q, a.q_stride_b, a.q_stride_s, a.q_stride_h = q.data_ptr(), *q.stride()[:3]
    a.rho, a.rho_stride_b, a.rho_stride_s, a.rho_stride_h = rho.data_ptr(), *rho.stride()[:3]
    a.k, a.k_stride_b, a.k_stride_s, a.k_stride_h = k.data_ptr(), *k.stride()[:3]
    a.v, a.v_stride_b, a.v_stride_s, a.v_stride_h = v.data_ptr(), *v.stride()[:3]
    a.out, a.out_stride_b, a.out_stride_s, a.out_stride_h = out.data_ptr(), *out.stride()[:3]
    a.window = W = args.window
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(i):
        st = lib.parallax_prefill(ctypes.byref(a), stream)
        if st != 0:
            plx._raise(st, lib)

    launch(0)
    torch.cuda.synchronize()
    cpu, parity = None, None
    if args.cpu_baseline:
        # sampled query rows of every (batch, head); their causal pairs scale
        # the oracle's time to the whole workload
        rng = np.random.default_rng(0)
        order = rng.permutation(S).astype(np.int32)
        hq, hr, hk, hv = (host_array(t) for t in (q, rho, k, v))
        threads = oracle.default_threads()
        secs, n, refs, done = 0.0, 24, [], 0
        while secs < args.cpu_seconds and done < S:  # grow the row sample to the budget
            batch = np.sort(order[done:done + n])
            t0 = time.perf_counter()
            refs.append((batch, oracle.prefill(hq, hr, hk, hv, scale, rows=batch,
                                               window=W, threads=threads)))
            secs += time.perf_counter() - t0
            done += n
            n *= 2
        rows = np.concatenate([r for r, _ in refs])
        ref = np.concatenate([o for _, o in refs], axis=1)
        ratio, rms = gate(out[:, rows.tolist()].double().cpu().numpy(), ref, 2e-2, 1e-2)
        parity = {"rows": f"{rows.size} sampled rows x all (batch, head)", "max_err_ratio": ratio,
                  "rel_rms": rms}
        seen = rows + 1 if W <= 0 else np.minimum(rows + 1, W)
        frac = float(np.sum(seen)) / causal_pairs(S, W)
        full = secs / frac
        cpu = {"value": prefill_flops(B, S, Hq, d, W) / full / 1e12, "unit": "TFLOP/s",
               "cores": threads, "kind": "oracle", "seconds_per_step": full,
               "sample": f"{rows.size} query rows x all (batch, head), fp64 streaming form; "
                         f"time scaled by causal pairs ({secs:.1f} s measured)"}
    secs = time_launches(torch, launch, 1, args.steps, args.warmup)
    per = secs / args.steps
    tflops = prefill_flops(B, S, Hq, d, W) / per / 1e12
    wtxt = f", local window {W}" if W > 0 else ""
    return {
        "metric": "Parallax causal prefill TFLOP/s (% of bf16 MFMA peak)", "value": round(tflops, 1),
        "unit": "TFLOP/s", "ms_per_step": per * 1e3, "dtype": "bf16",
        "config": {"workload": f"causal prefill: batch 4, seq 8192, {Hq} query / {Hkv} KV heads, "
                               f"d {d}, bf16 q/rho/k/v, fp32 out{wtxt}", "batch": B, "seq_len": S,
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d, "window": W},
        "mfma_util": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "tokens_per_s": B * S / per,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_for("prefill") if (W, d, Hq, Hkv) == (0, 128, 16, 8) else None},
        "parity": parity, "cpu_baseline": cpu,
    }


def prefill_bwd_flops(B, S, Hq, d, window=0):
    """Algorithmic flops of the backward pass: per causal (query, key) pair
    and query head, eight products of 2*d flops each -- the scores q.k and
    probe projections rho.k recomputed, u = dout.v, and the gradient sums
    into dv, dk (from ds and from dt), dq and drho."""
    return 8 * 2 * d * causal_pairs(S, window) * B * Hq


def run_prefill_bwd(args, torch, plx):
    import ctypes
    import numpy as np
    import oracle
    from parallax_local_linear_decode_amd.workloads import (host_array, prefill_dout,
                                                            prefill_inputs)
    B, S, Hq, Hkv, d = 4, 8192, args.q_heads, args.kv_heads, args.head_dim
    W = args.window
    dev = torch.device("cuda:0")
    q, rho, k, v, scale = prefill_inputs(B, S, Hq, Hkv, d, seed=0, device=dev)
    dout = prefill_dout(B, S, Hq, d, seed=1, device=dev)
    out, lse, rmean, o_sa = plx.parallax_prefill(q, rho, k, v, scale=scale, window=W,
                                                 return_stats=True)
    dq = torch.empty((B, S, Hq, d), dtype=torch.float32, device=dev)
    drho = torch.empty_like(dq)
    dk = torch.empty((B, S, Hkv, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    lib = plx.load_library()
    a = plx._backward_args(q, rho, k, v, dout, out, o_sa, lse, rmean, dq, drho, dk, dv, scale,
                           True, W)
    need = ctypes.c_size_t(0)
    if lib.parallax_prefill_backward_workspace_size(ctypes.byref(a), ctypes.byref(need)) != 0:
        raise SystemExit(plx.parallax_last_error())
    ws = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(i):
        st = lib.parallax_prefill_backward(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()),
                                           ws.numel(), stream)
        if st != 0:
            plx._raise(st, lib)

    launch(0)
    torch.cuda.synchronize()
    # parity of the timed data: sampled rows' dq / drho, the last 64 keys'
    # dk / dv (exact from rows S-64..S-1), on sequence 0 and every head
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.integers(0, S - 64, 8), np.arange(S - 64, S)]))
    rows = rows.astype(np.int32)
    sub = [host_array(t[:1]) for t in (q, rho, k, v, dout)]
    r_dq, r_drho, r_dk, r_dv = oracle.prefill_backward(*sub, scale, rows=rows, window=W)
    sel = torch.as_tensor(rows, dtype=torch.long)
    parity = {}
    for name, got, ref in (("dq", dq[:1, sel], r_dq), ("drho", drho[:1, sel], r_drho),
                           ("dk", dk[:1, S - 64:], r_dk[:, S - 64:]),
                           ("dv", dv[:1, S - 64:], r_dv[:, S - 64:])):
        ratio, rms = gate(got.double().cpu().numpy(), ref, TAU_BWD, 1e-2)
        parity[name] = {"max_err_ratio": ratio, "rel_rms": rms}
    flops = prefill_bwd_flops(B, S, Hq, d, W)
    cpu = None
    if args.cpu_baseline:
        # the oracle's backward over a growing sample of query rows of every
        # (batch, head); its time is scaled by the causal pairs covered
        hq = [host_array(t) for t in (q, rho, k, v, dout)]
        threads = oracle.default_threads()
        order = rng.permutation(S).astype(np.int32)
        secs, n, done, seen = 0.0, 8, 0, 0
        while secs < args.cpu_seconds and done < S:
            batch = np.sort(order[done:done + n])
            t0 = time.perf_counter()
            oracle.prefill_backward(*hq, scale, rows=batch, window=W, threads=threads)
            secs += time.perf_counter() - t0
            seen += int(np.sum(batch + 1 if W <= 0 else np.minimum(batch + 1, W)))
            done += n
            n *= 2
        full = secs * causal_pairs(S, W) / seen
        cpu = {"value": flops / full / 1e12, "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "seconds_per_step": full,
               "sample": f"{done} query rows x all (batch, head), fp64 chain rule; time "
                         f"scaled by causal pairs ({secs:.1f} s measured)"}
    secs = time_launches(torch, launch, 1, args.steps, args.warmup)
    per = secs / args.steps
    tflops = flops / per / 1e12
    wtxt = f", local window {W}" if W > 0 else ""
    return {
        "metric": "Parallax causal prefill backward TFLOP/s (% of bf16 MFMA peak)",
        "value": round(tflops, 1), "unit": "TFLOP/s", "ms_per_step": per * 1e3, "dtype": "bf16",
        "config": {"workload": "causal prefill backward (dq, drho, dk, dv): batch 4, seq 8192, "
                               f"{Hq} query / {Hkv} KV heads, d {d}, bf16 inputs and dout{wtxt}",
                   "batch": B, "seq_len": S, "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": d, "window": W},
        "mfma_util": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "tokens_per_s": B * S / per,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (traffic_for("prefill_bwd")
                                 if (W, d, Hq, Hkv) == (0, 128, 16, 8) else None)},
        "parity": parity, "cpu_baseline": cpu,
    }


def gate(gpu, ref, tau, rms):
    """Parity of GPU results with the oracle's: max |g - r| / (1 + |r|) <= tau
    and ||g - r|| / ||r|| <= rms, or the run stops without reporting."""
    import numpy as np
    ratio = float(np.max(np.abs(gpu - ref) / (1 + np.abs(ref))))
    r = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"parity vs oracle: max err ratio {ratio:.3e}, rel-RMS {r:.3e}")
    if not (ratio <= tau and r <= rms) or not np.all(np.isfinite(gpu)):
        raise SystemExit(f"parity gate failed (ratio {ratio:.3e}, rel-RMS {r:.3e})")
    return ratio, r


def label_cpu_baselines(rec, cpu_model):
    """Name the host CPU in every oracle baseline of a record, nested ones too."""
    if isinstance(rec, dict):
        for k, v in rec.items():
            if k == "cpu_baseline" and isinstance(v, dict):
                v.setdefault("cpu_model", cpu_model)
            else:
                label_cpu_baselines(v, cpu_model)
    elif isinstance(rec, list):
        for v in rec:
            label_cpu_baselines(v, cpu_model)


def host_info():
    """The host the oracle baselines run on: CPU model and usable cores."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cores": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="suite",
                    choices=["suite", "decode", "paged", "prefill", "prefill_bwd", "lla", "qr_proj",
                             "sweep", "copy", "issue", "sdpa"])
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--ctx", type=int, default=4096)
    ap.add_argument("--split", type=int, default=0, help="split_tokens (0 = library choice)")
    ap.add_argument("--window", type=int, default=0,
                    help="local window for decode / prefill (0 = full attention)")
    ap.add_argument("--head-dim", type=int, default=128, choices=(64, 128),
                    help="head dim (workloads prefill and prefill_bwd)")
    ap.add_argument("--q-heads", type=int, default=16, help="query heads (prefill, prefill_bwd)")
    ap.add_argument("--kv-heads", type=int, default=8, help="KV heads (prefill, prefill_bwd)")
    ap.add_argument("--tokens", type=int, default=8, help="token rows (workload qr_proj)")
    ap.add_argument("--model-dim", type=int, default=2048, help="model dim (workload qr_proj)")
    ap.add_argument("--lla-lambda", type=float, default=0.5, help="LLA ridge term (workload lla)")
    ap.add_argument("--lla-iters", type=int, default=16, help="LLA CG iterations (workload lla)")
    ap.add_argument("--cold-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time budget of the headline CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if "RANK" in os.environ and os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)
    import torch
    sys.path.insert(0, ROOT)
    import parallax_local_linear_decode_amd as plx
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    plx.load_library()
    runner = {"suite": run_suite, "decode": run_decode, "paged": run_paged, "sweep": run_sweep,
              "copy": run_copy, "prefill": run_prefill,
              "prefill_bwd": run_prefill_bwd, "lla": run_lla,
              "qr_proj": run_qr_proj, "issue": run_issue,
              "sdpa": run_sdpa}.get(args.workload)
    if runner is None:
        raise SystemExit(f"workload {args.workload} is not available")
    rec = runner(args, torch, plx)
    line = {"metric": rec["metric"], "value": rec["value"], "unit": rec["unit"], "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": rec["dtype"], "data": "synthetic (seeded N(0,1) q/k/v, N(0,0.1^2) rho)",
            "config": rec["config"]}
    line["roofline"] = rec["roofline"]
    line["cpu_baseline"] = rec["cpu_baseline"]
    for k, v in rec.items():  # the workload's own figures and sub-records
        if k not in line:
            line[k] = v
    label_cpu_baselines(line, host_info()["cpu_model"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
