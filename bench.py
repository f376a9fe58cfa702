#!/usr/bin/env python3
"""Benchmark of shared-history cross-attention on one MI355X.

One step = one xattn_forward call over one batch of synthetic inputs resident
in HBM.  For small batches (at most 16 requests, model width at most 256)
that is a single kernel that plans the batch, projects its queries and runs
the attention; for batches of short memories on a 256-wide model it is the
short-memory kernel; otherwise it is the projection GEMM (which also runs the
planner) followed by the attention kernel.  Default workload: the long
history (4 requests of 16384 memory rows, d = 512 as 8 heads x 64, 512
candidates x 3 query tokens, K = V = H, bf16), the largest single-GPU batch
by work: the ReST length and width scaling point (ReST reading note, s.5.3).

Prints one JSON line with the whole-step throughput (candidate-queries/s),
the dominant kernel's roofline fraction (its average launch duration measured
with HIP events on the launch stream), the fp64 CPU oracle timed on a bounded
sample of the same workload on this host's cores, and the same forward
measurement for the other benchmark batches (field "other_workloads").

Timing.  Every timed loop makes C-ABI calls whose arguments were marshalled
once (BoundCall), so host-side checks add nothing between kernels.  Before
the W warm-up steps the step runs untimed for --settle-ms so that the clocks
have left their idle state; the K timed steps follow the W warm-up steps.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

CONFIGS = ("rest", "long", "transx", "ragged", "tiny")
_ATTN_SRC = ["shared_history_candidate_amd/csrc/attn_bf16.hip",
             "shared_history_candidate_amd/csrc/lds_dma.h",
             "shared_history_candidate_amd/csrc/plan_wave.h",
             "shared_history_candidate_amd/csrc/xcd_order.h",
             "shared_history_candidate_amd/csrc/common.h"]
KERNEL_SOURCES = {"fused": _ATTN_SRC, "attention": _ATTN_SRC, "prefix": _ATTN_SRC,
                  "fused_prefix": _ATTN_SRC,
                  "backward": ["shared_history_candidate_amd/csrc/bwd_bf16.hip"] + _ATTN_SRC,
                  "output": ["shared_history_candidate_amd/csrc/gemm_bf16.hip",
                             "shared_history_candidate_amd/csrc/output_bf16.hip",
                             "shared_history_candidate_amd/csrc/common.h"],
                  "projection": ["shared_history_candidate_amd/csrc/gemm_bf16.hip",
                                 "shared_history_candidate_amd/csrc/plan_device.h",
                                 "shared_history_candidate_amd/csrc/common.h"],
                  "short": ["shared_history_candidate_amd/csrc/short_bf16.hip",
                            "shared_history_candidate_amd/csrc/common.h"]}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--config", default="long", choices=CONFIGS)
    p.add_argument("--settle-ms", type=float, default=300.0,
                   help="untimed run of the step before the warm-up steps (clock ramp)")
    p.add_argument("--only", action="store_true",
                   help="measure --config alone (no other_workloads field)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--stage", default="attention",
                   choices=("attention", "output", "prefix", "backward", "backward_prefix",
                            "codec"),
                   help="attention: the hot path (xattn_forward, the default); output: the "
                        "gate and output projection of Eq. (7) alone (xattn_output); prefix: "
                        "the forward with per-candidate prefix lengths (xattn_forward_prefix); "
                        "backward: the gradients of the attention (xattn_backward); "
                        "backward_prefix: the same with per-candidate prefix lengths; codec: "
                        "the forward over a coded memory at --codec-bits bits per coordinate "
                        "(xattn_forward_codec)")
    p.add_argument("--codec-bits", type=float, default=4.5,
                   help="average bits per coordinate of the coded memory (stage codec)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="run only a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--ingest-counters", metavar="DIR",
                   help="write profiles/counters_*_<config>.json from rocprofv3 --pmc runs in DIR "
                        "(fetch/, write/, calib_fetch/, calib_write/)")
    p.add_argument("--micro", action="store_true",
                   help="run only the unit micro-benchmarks (achievable MFMA/exp/VALU/LDS/HBM)")
    return p.parse_args()


def micro():
    """Achievable rates of the units that bound the fused kernel (one JSON line)."""
    import ctypes
    import torch
    from shared_history_candidate_amd import xattn as X
    L = X.lib()
    L.xattn_micro_run.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    L.xattn_micro_run.restype = ctypes.c_float
    L.xattn_micro_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p]
    L.xattn_micro_copy.restype = ctypes.c_float
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    clk = 2.4e9
    blocks = cus * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {"cus": cus, "assumed_clock_ghz": clk / 1e9}
    iters = 2000
    ms = L.xattn_micro_run(0, blocks, iters, 5, ctypes.c_void_p(out.data_ptr()), st)
    fl = blocks * 4 * iters * 8 * 32768.0
    res["mfma_bf16_tflops"] = fl / (ms * 1e-3) / 1e12
    for kind, name, per in ((1, "exp", 16), (2, "fma", 16)):
        ms = L.xattn_micro_run(kind, blocks, iters, 5, ctypes.c_void_p(out.data_ptr()), st)
        ops = blocks * 256 * iters * per
        res[name + "_per_cu_per_clk"] = ops / (ms * 1e-3) / (cus * clk)
    for kind, name, nbytes in ((3, "lds_b64", 16), (4, "lds_b128", 16), (5, "lds_tr16_b64", 16)):
        ms = L.xattn_micro_run(kind, blocks, iters, 5, ctypes.c_void_p(out.data_ptr()), st)
        b = blocks * 256 * iters * float(nbytes)
        res[name + "_bytes_per_cu_per_clk"] = b / (ms * 1e-3) / (cus * clk)
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b2 = torch.empty_like(a)
    ms = L.xattn_micro_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b2.data_ptr()), n, 10, st)
    res["hbm_copy_gbs"] = 2.0 * n / (ms * 1e-3) / 1e9
    print(json.dumps({k: (round(v, 3) if isinstance(v, float) else v) for k, v in res.items()}))


def kernel_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


# Kernel names (regular expressions over the demangled or mangled names) of
# the kernels a step can run: the single launch of a small batch (attention
# kernel that projects its own queries: flags PROJ=1, CUT=0, or CUT=1 with
# per-candidate prefix lengths), the projection GEMM and the attention kernel
# over its output (PROJ=0; CUT=1 with prefix lengths; a last flag set for the
# head-pair form of 32-wide heads), or the short-memory kernel.
KERNEL_NAMES = {
    "fused": r"attn_bf16_kernel(<\d+, \d+, \d+, \w+, true, false(, \w+)?>|"
             r"ILi\d+ELi\d+ELi\d+ELb[01]ELb1ELb0E)",
    "fused_prefix": r"attn_bf16_kernel(<\d+, \d+, \d+, \w+, true, true(, \w+)?>|"
                    r"ILi\d+ELi\d+ELi\d+ELb[01]ELb1ELb1E)",
    "attention": r"attn_bf16_kernel(<\d+, \d+, \d+, \w+, false, false(, \w+)?>|"
                 r"ILi\d+ELi\d+ELi\d+ELb[01]ELb0ELb0E)",
    "prefix": r"attn_bf16_kernel(<\d+, \d+, \d+, \w+, false, true(, \w+)?>|"
              r"ILi\d+ELi\d+ELi\d+ELb[01]ELb0ELb1E)",
    "projection": r"prep_kernel",
    "short": r"short_bf16_kernel"}


def traffic_for(kernel, config):
    """HBM bytes per launch of a kernel from committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for
    a plain copy of known size), or None when absent or taken on a different
    kernel source."""
    path = os.path.join(ROOT, "profiles", "counters_%s_%s.json" % (kernel, config))
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    if c.get("kernel_source_sha") != kernel_sha(kernel):
        return None
    return round(c["fetch_kib"] * 1024.0 * c["fetch_calibration"] +
                 c["write_kib"] * 1024.0 * c["write_calibration"], 1)


def _counter_means(csv_path, name_re, counter):
    """Average per dispatch of one counter over the dispatches of kernels
    whose name matches name_re (rocprofv3 --pmc CSV), or None if none ran."""
    import csv
    import re
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if re.search(name_re, r["Kernel_Name"]) and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        return None, 0
    return sum(per.values()) / len(per), len(per)


def ingest_counters(d, config, calib_mib):
    """Turn four rocprofv3 --pmc runs under directory d (fetch/, write/:
    this benchmark; calib_fetch/, calib_write/: --calib-copy-mib) into
    profiles/counters_<kernel>_<config>.json for both kernels."""
    csvf = lambda sub: os.path.join(d, sub, "run_counter_collection.csv")
    known = calib_mib * (1 << 20)
    cf, _ = _counter_means(csvf("calib_fetch"), "copy_kernel", "FETCH_SIZE")
    cw, _ = _counter_means(csvf("calib_write"), "copy_kernel", "WRITE_SIZE")
    for kernel, part in KERNEL_NAMES.items():
        f, nf = _counter_means(csvf("fetch"), part, "FETCH_SIZE")
        w, nw = _counter_means(csvf("write"), part, "WRITE_SIZE")
        if f is None or w is None:
            continue   # this workload does not run that kernel
        out = {"kernel": part, "workload": config, "fetch_kib": round(f, 1),
               "write_kib": round(w, 1), "dispatches": [nf, nw],
               "fetch_calibration": round(known / (cf * 1024.0), 4),
               "write_calibration": round(known / (cw * 1024.0), 4),
               "calibration_copy_bytes": known,
               "kernel_source_sha": kernel_sha(kernel)}
        path = os.path.join(ROOT, "profiles", "counters_%s_%s.json" % (kernel, config))
        json.dump(out, open(path, "w"), indent=1)
        print(path, json.dumps(out))


def roofline(flops, nbytes, ms, dtype):
    """Bound of a kernel by its arithmetic intensity against the ridge point,
    and the achieved rate against that bound's MI355X peak."""
    peak_flops = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if dtype != "bf16":
        bound = "alu"
    else:
        bound = "mfma" if flops / nbytes >= ridge else "hbm"
    if bound == "hbm":
        achieved, peak, unit = nbytes / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = flops / (ms * 1e-3) / 1e12, peak_flops, "TFLOP/s"
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 5)}


def cpu_baseline(wl, target_s, stage="attention", seed=0):
    """The fp64 oracle as it stands, timed on this host on a bounded sample of
    the workload's query rows (grown until it takes about target_s).  For the
    output stage the sample is whole candidates (all their query slots); the
    prefix stage runs the oracle with the same prefix lengths as the GPU."""
    import numpy as np
    import oracle
    from shared_history_candidate_amd import workloads as W
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    rng = np.random.default_rng(1)
    kv_len = (W.prefix_lengths(wl, seed + 3, out_of_range=False)
              if stage in ("prefix", "backward_prefix") else None)
    if stage in ("backward", "backward_prefix"):
        return _cpu_baseline_backward(wl, target_s, seed, threads,
                                      kv_len if stage == "backward_prefix" else None)
    if stage == "output":
        wgo, wo = W.output_weights(wl, seed + 1)
        O_in = W.attention_like(wl, seed + 2)
    n = min(wl.rows, 64)
    done, elapsed, runs = 0, 0.0, 0
    while True:
        rows = np.sort(rng.choice(wl.rows, size=n, replace=False)) if n < wl.rows else None
        t0 = time.perf_counter()
        if stage == "output":
            c = np.unique(rows // wl.q) if rows is not None else np.arange(wl.total_cand)
            oracle.output(wl.Z[c], wgo, O_in[c], wo, wl.q)
            n = len(c) * wl.q
        else:
            oracle.forward(wl.cu_kv, wl.cu_cand, wl.q, wl.heads, wl.Z, wl.wt, wl.K, wl.V,
                           rows=rows, kv_len=kv_len)
        dt = time.perf_counter() - t0
        done += n
        elapsed += dt
        runs += 1
        if elapsed >= target_s:
            break
        if n < wl.rows:
            per_row = dt / n
            n = int(min(wl.rows, max(n * 2, (target_s - elapsed) / max(per_row, 1e-9))))
    if runs == 1 and n == wl.rows:
        sample = "all %d query rows once" % wl.rows
    else:
        sample = "%d query rows in %d oracle calls (random rows of the same batch, full rows " \
                 "of the batch when it fits)" % (done, runs)
    return {"value": done / elapsed, "unit": "candidate-queries/s", "cores": threads,
            "kind": "oracle", "sample": sample, "seconds": round(elapsed, 2)}


def _cpu_baseline_backward(wl, target_s, seed, threads, kv_len=None):
    """The oracle's backward on the batch's first k requests (a gradient of a
    memory needs every query row of its request), k doubled until the run
    takes about target_s; rows of those requests per second."""
    import numpy as np
    import oracle
    from shared_history_candidate_amd import workloads as W
    dO = W.output_grad(wl, seed + 4).reshape(-1, wl.d)
    k, done, elapsed, runs = 1, 0, 0.0, 0
    while True:
        cu_kv = wl.cu_kv[:k + 1]
        cu_c = wl.cu_cand[:k + 1]
        rows = int(cu_c[-1]) * wl.q
        kv = int(cu_kv[-1])
        t0 = time.perf_counter()
        oracle.backward(cu_kv, cu_c, wl.q, wl.heads, wl.Z.reshape(-1, wl.d)[:rows], wl.wt,
                        wl.K[:kv], wl.V[:kv] if wl.V is not None else None, dO[:rows],
                        kv_len=kv_len[:int(cu_c[-1])] if kv_len is not None else None)
        dt = time.perf_counter() - t0
        done += rows
        elapsed += dt
        runs += 1
        if elapsed >= target_s or k >= wl.R:
            break
        k = min(wl.R, k * 2)
    return {"value": done / elapsed, "unit": "candidate-queries/s", "cores": threads,
            "kind": "oracle", "seconds": round(elapsed, 2),
            "sample": "backward of the first requests of the batch (%d query rows in %d oracle "
                      "calls, up to %d of %d requests)" % (done, runs, k, wl.R)}


def calib_copy(mib):
    """A plain device copy of mib MiB (the library's copy_kernel, 16-byte
    loads and stores): the known-size reference for the HBM byte counters."""
    import ctypes
    import torch
    from shared_history_candidate_amd import xattn as X
    L = X.lib()
    L.xattn_micro_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_void_p]
    L.xattn_micro_copy.restype = ctypes.c_float
    n = mib * (1 << 20)
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ms = L.xattn_micro_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), n, 5, st)
    L.xattn_micro_half_line_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
    L.xattn_micro_half_line_read.restype = ctypes.c_float
    out = torch.empty(256 * 8 * 256, dtype=torch.float32, device="cuda")
    ms_half = L.xattn_micro_half_line_read(ctypes.c_void_p(a.data_ptr()), n, 5,
                                           ctypes.c_void_p(out.data_ptr()), st)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n,
                      "launches": 6, "ms_per_copy": round(ms, 4),
                      "copy_gbs": round(2.0 * n / (ms * 1e-3) / 1e9, 1),
                      "half_line_read_bytes": n // 2, "half_line_launches": 6,
                      "ms_per_half_line_read": round(ms_half, 4)}))


def settle(step, stream, ms):
    """Run step untimed for about ms milliseconds of device time (clocks
    leave their idle state; the timed loops then see a steady clock)."""
    import torch
    if ms <= 0:
        return
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    done, n = 0.0, 4
    while done < ms:
        a.record(stream)
        for _ in range(n):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        dt = a.elapsed_time(b)
        done += dt
        n = min(4096, n * 2)


def timed_loop(fn, stream, n):
    """Device time of n back-to-back calls of fn between one HIP event pair on
    the launch stream, per call (an event pair per call would add its own
    ~1-2 us to every call)."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def forward_setup(ctx, wl, t, ws, O, stream, cut=None):
    """Bound calls of the forward step and of its kernels alone for one batch:
    (step, kernels) with kernels = {name: (bound call, flops, bytes)} for the
    kernels a step launches, and the path taken."""
    import torch
    from shared_history_candidate_amd import xattn as X
    path = ctx.forward_path(wl.R, wl.total_cand, wl.total_kv, wl.heads)
    launches = ctx.forward_launches(wl.R, wl.total_cand, wl.total_kv, wl.heads)
    step = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads,
                       O=O, workspace=ws, stream=stream, cand_kv_len=cut, bind=True)
    step()   # the plan the kernels alone read below
    if cut is None and path == X.PATH_SHORT:
        # one kernel plans the batch, projects and attends: the path's work
        kernels = {"short": (step, wl.flops(), wl.bytes())}
    elif cut is None and launches == 1:
        # the attention kernel plans the batch and projects its own queries
        kernels = {"fused": (step, wl.flops(), wl.bytes())}
    elif launches == 1:
        # the same single launch with per-candidate prefix lengths: the
        # projection's work and the visible rows' attention, with Z and W_Q
        # read in place of Q
        kv_arg = cut.cpu().numpy()
        b = 2 if wl.dtype == "bf16" else 4
        kernels = {"fused_prefix": (step, wl.flops_projection() + wl.flops_attention(kv_arg),
                                    wl.bytes_attention(kv_arg) + b * wl.q * wl.d * wl.d)}
    else:
        Qbuf = torch.empty_like(O)
        proj = ctx.project(t["Z"], t["W_Q"], Q=Qbuf, stream=stream, bind=True)
        proj()
        attn = ctx.attend_q(Qbuf, t["K"], t["V"], t["cu_kv"], t["cu_cand"], wl.heads, ws, O=O,
                            stream=stream, cand_kv_len=cut, bind=True)
        attn.keep = Qbuf   # the bound call reads this buffer
        kv_arg = cut.cpu().numpy() if cut is not None else None
        kernels = {("prefix" if cut is not None else "attention"):
                       (attn, wl.flops_attention(kv_arg), wl.bytes_attention(kv_arg)),
                   "projection": (proj, wl.flops_projection(), wl.bytes_projection())}
    return step, kernels, path


def measure_forward(ctx, wl, t, ws, O, stream, steps, warmup, settle_ms, config_name, cut=None):
    """ms per forward step and the roofline entry of its dominant kernel
    (the other kernel, if any, in other_kernel)."""
    step, kernels, path = forward_setup(ctx, wl, t, ws, O, stream, cut)
    settle(step, stream, settle_ms)
    for _ in range(warmup):
        step()
    ms_per_step = timed_loop(step, stream, steps)
    entries = {}
    for name, (fn, flops, nbytes) in kernels.items():
        kms = ms_per_step if fn is step else timed_loop(fn, stream, steps)
        entries[name] = dict(roofline(flops, nbytes, kms, wl.dtype), kernel_ms=round(kms, 5),
                             algorithmic_flops=flops, algorithmic_bytes=nbytes,
                             traffic=traffic_for(name, config_name), kernel=name)
    dominant = max(entries, key=lambda k: entries[k]["kernel_ms"])
    roof = dict(entries[dominant])
    others = [v for k, v in entries.items() if k != dominant]
    roof["other_kernel"] = others[0] if others else None
    if roof["kernel_ms"] > ms_per_step * 1.001:
        raise RuntimeError("kernel time %.5f ms exceeds the step time %.5f ms: the timing is "
                           "not trustworthy" % (roof["kernel_ms"], ms_per_step))
    return ms_per_step, roof, path


def other_workloads(args, X, W, torch):
    """The forward measurement of every other benchmark batch (shorter loops,
    no CPU baseline): one small dict per workload."""
    out = []
    stream = torch.cuda.current_stream()
    for name in CONFIGS:
        if name in (args.config, "tiny"):
            continue
        wl = W.make(name, args.seed)
        ctx = X.XAttn(wl.d, wl.q, wl.dtype, wl.kv_mode)
        t = X.to_device(wl)
        ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
        O = torch.empty((wl.total_cand, wl.q, wl.d), dtype=ctx.torch_dtype, device="cuda")
        n = max(20, min(args.steps, 200))
        ms, roof, path = measure_forward(ctx, wl, t, ws, O, stream, n, max(args.warmup, 5),
                                         args.settle_ms / 3, name)
        out.append({"workload": wl.name, "steps": n, "ms_per_step": round(ms, 5),
                    "value": round(wl.rows / (ms * 1e-3), 1), "unit": "candidate-queries/s",
                    "kernel": roof["kernel"], "kernel_ms": roof["kernel_ms"],
                    "bound": roof["bound"], "achieved": roof["achieved"],
                    "unit_roofline": roof["unit"], "frac": roof["frac"],
                    "traffic": roof["traffic"]})
        print("bench: %s %.4f ms/step, %s %.4f ms (%.1f %% of %s peak)" %
              (wl.name, ms, roof["kernel"], roof["kernel_ms"], 100 * roof["frac"], roof["bound"]),
              file=sys.stderr, flush=True)
        del ctx, t, ws, O
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(requests shard across GPUs with no exchange). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.ingest_counters:
        ingest_counters(args.ingest_counters, args.config, args.calib_copy_mib or 256)
        return
    if args.calib_copy_mib:
        calib_copy(args.calib_copy_mib)
        return
    if args.micro:
        micro()
        return

    import numpy as np
    import torch
    from shared_history_candidate_amd import workloads as W
    from shared_history_candidate_amd import xattn as X

    wl = W.make(args.config, args.seed)
    print("bench: workload %s R=%d rows=%d total_kv=%d d=%d heads=%d" %
          (wl.name, wl.R, wl.rows, wl.total_kv, wl.d, wl.heads), file=sys.stderr, flush=True)
    ctx = X.XAttn(wl.d, wl.q, wl.dtype, wl.kv_mode)
    t = X.to_device(wl)
    ws = ctx.alloc_workspace(wl.R, wl.total_cand, wl.heads)
    O = torch.empty((wl.total_cand, wl.q, wl.d), dtype=ctx.torch_dtype, device="cuda")
    stream = torch.cuda.current_stream()
    kv_len = None
    others = None

    if args.stage in ("attention", "prefix"):
        cl = None
        if args.stage == "prefix":
            # per-candidate prefix lengths: sorted draws from U{0..L_r} per request
            kv_len = W.prefix_lengths(wl, args.seed + 3, out_of_range=False)
            cl = torch.from_numpy(kv_len).to("cuda")
        ms_per_step, roof, path = measure_forward(ctx, wl, t, ws, O, stream, args.steps,
                                                  args.warmup, args.settle_ms, args.config, cl)
        print("bench: %d steps, %.4f ms/step; %s %.4f ms per launch" %
              (args.steps, ms_per_step, roof["kernel"], roof["kernel_ms"]),
              file=sys.stderr, flush=True)
        if roof["other_kernel"]:
            print("bench: %s %.4f ms per launch" % (roof["other_kernel"]["kernel"],
                                                   roof["other_kernel"]["kernel_ms"]),
                  file=sys.stderr, flush=True)
        if path == X.PATH_SHORT and args.stage == "attention":
            # the same kernel over the stored plan (no planning), for reference
            att = ctx.forward(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"], t["cu_cand"],
                              wl.heads, O=O, workspace=ws, stream=stream, plan=False, bind=True)
            print("bench: short-memory kernel over a stored plan %.4f ms" %
                  timed_loop(att, stream, args.steps), file=sys.stderr, flush=True)
        if args.stage == "attention" and not args.only:
            others = other_workloads(args, X, W, torch)
    else:
        if args.stage == "output":
            wgo, wo = W.output_weights(wl, args.seed + 1)
            dt = ctx.torch_dtype
            up = lambda a: torch.from_numpy(a).to("cuda").to(dt).contiguous()
            Wgo_d, Wo_d, O_in = up(wgo), up(wo), up(W.attention_like(wl, args.seed + 2))

            def step():
                ctx.output(t["Z"], Wgo_d, O_in, Wo_d, ws, Y=O, stream=stream)
        elif args.stage in ("backward", "backward_prefix"):
            dO_d = torch.from_numpy(W.output_grad(wl, args.seed + 4)).to("cuda").to(
                ctx.torch_dtype).contiguous()
            kv_len = (W.prefix_lengths(wl, args.seed + 3, out_of_range=False)
                      if args.stage == "backward_prefix" else None)
            cl = torch.from_numpy(kv_len).to("cuda") if kv_len is not None else None
            grads = ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], dO_d, t["cu_kv"],
                                 t["cu_cand"], wl.heads, cand_kv_len=cl)
            bws = torch.empty(max(ctx.backward_workspace_size(wl.R, wl.total_cand, wl.total_kv,
                                                              wl.heads), 256),
                              dtype=torch.uint8, device="cuda")

            def step():
                ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], dO_d, t["cu_kv"], t["cu_cand"],
                             wl.heads, workspace=bws, out=grads, stream=stream, cand_kv_len=cl)

            # the training pair: a forward that keeps the normalisers, and the
            # backward that reuses them (bf16 only)
            train_pair = wl.dtype == "bf16"
            if train_pair:
                O_tr, lse_tr = ctx.forward_train(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"],
                                                 t["cu_cand"], wl.heads, workspace=ws,
                                                 cand_kv_len=cl)

                def step_train_fwd():
                    ctx.forward_train(t["Z"], t["W_Q"], t["K"], t["V"], t["cu_kv"],
                                      t["cu_cand"], wl.heads, O=O_tr, lse=lse_tr, workspace=ws,
                                      stream=stream, cand_kv_len=cl)

                def step_saved():
                    ctx.backward(t["Z"], t["W_Q"], t["K"], t["V"], dO_d, t["cu_kv"],
                                 t["cu_cand"], wl.heads, workspace=bws, out=grads,
                                 stream=stream, cand_kv_len=cl, O=O_tr, lse=lse_tr)
        elif args.stage == "codec":
            # memory published as codes + norms (encoded once, outside the step)
            # codebooks fitted by the library on a sample of the memory rows
            # (offline calibration, not part of a step)
            budget = int(round(args.codec_bits * wl.d_h / 32.0)) * 32
            rng = np.random.default_rng(args.seed + 5)
            pick = np.sort(rng.choice(wl.total_kv, min(wl.total_kv, 4096), replace=False))
            mem = [wl.K] + ([wl.V] if wl.V is not None else [])
            books = [X.codec_fit(m[pick], wl.heads, budget) for m in mem]
            books += books[:1] * (2 - len(books))
            cbs = [X.Codebook(b["bits"], b["center"], b["half"], b["rot"], b["budget"])
                   for b in books]
            kc, kn = ctx.codec_encode(cbs[0], t["K"])
            vc, vn = ctx.codec_encode(cbs[1], t["V"]) if t["V"] is not None else (None, None)
            cbv = cbs[1] if t["V"] is not None else None
            Wr = ctx.codec_fold(cbs[0], t["W_Q"])
            codec_bytes = (kc.numel() + kn.numel()) * 4 * (2 if cbv is not None else 1)
            # a workspace with room for the decoded memory: the memory is decoded
            # once per call where the short-memory kernel does not take the batch
            cws = torch.empty(max(ctx.codec_workspace_size(wl.R, wl.total_cand, wl.total_kv,
                                                           wl.heads), 256),
                              dtype=torch.uint8, device="cuda")

            def step():
                ctx.forward_codec(cbs[0], cbv, t["Z"], Wr, kc, kn, vc, vn, t["cu_kv"],
                                  t["cu_cand"], wl.heads, O=O, workspace=cws, stream=stream)

            def step_lds():
                ctx.forward_codec(cbs[0], cbv, t["Z"], Wr, kc, kn, vc, vn, t["cu_kv"],
                                  t["cu_cand"], wl.heads, O=O, workspace=ws, stream=stream)

        # these stages are timed as one unit per call (several launches; the
        # per-kernel split is in the kernel traces)
        step()
        settle(step, stream, args.settle_ms)
        for _ in range(args.warmup):
            step()
        ms_per_step = timed_loop(step, stream, args.steps)
        print("bench: %d steps, %.4f ms/step" % (args.steps, ms_per_step), file=sys.stderr,
              flush=True)

        def entry(kernel, flops, nbytes, ms):
            return dict(roofline(flops, nbytes, ms, wl.dtype), kernel_ms=round(ms, 5),
                        algorithmic_flops=flops, algorithmic_bytes=nbytes,
                        traffic=traffic_for(kernel, args.config), kernel=kernel,
                        other_kernel=None)

        if args.stage in ("backward", "backward_prefix"):
            roof = entry("backward", wl.flops_backward(kv_len), wl.bytes_backward(), ms_per_step)
            if train_pair:
                tf_ms = timed_loop(step_train_fwd, stream, args.steps)
                sv_ms = timed_loop(step_saved, stream, args.steps)
                print("bench: training forward (keeps lse) %.4f ms; backward from the stored "
                      "statistics %.4f ms" % (tf_ms, sv_ms), file=sys.stderr, flush=True)
                roof["training_forward_ms"] = round(tf_ms, 5)
                roof["saved_statistics_backward_ms"] = round(sv_ms, 5)
        elif args.stage == "codec":
            # bytes count codes + norms for the memory.  For reference, the same
            # call with the plain workspace (each memory tile reconstructed in
            # LDS by every query tile).
            lds_ms = timed_loop(step_lds, stream, args.steps)
            print("bench: codec forward %.4f ms (memory %.2f MB coded vs %.2f MB bf16); "
                  "with the plain workspace %.4f ms" %
                  (ms_per_step, codec_bytes / 1e6,
                   wl.total_kv * wl.d * 2 * (2 if wl.kv_mode == "separate" else 1) / 1e6,
                   lds_ms), file=sys.stderr, flush=True)
            b = 2.0 * (2 * wl.rows * wl.d + wl.q * wl.d * wl.d) + codec_bytes
            roof = entry("codec", wl.flops(), b, ms_per_step)
        else:
            roof = entry("output", wl.flops_output(), wl.bytes_output(), ms_per_step)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds, args.stage, args.seed)

    value = wl.rows / (ms_per_step * 1e-3)
    line = {
        "metric": "candidate-queries scored/sec", "value": round(value, 1),
        "unit": "candidate-queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "requests": wl.R, "candidates": wl.total_cand,
                   "query_tokens": wl.q, "memory_rows": wl.total_kv, "d": wl.d,
                   "heads": wl.heads, "kv_mode": wl.kv_mode, "seed": args.seed,
                   "stage": {"attention": "forward (attention path)",
                             "output": "output gate and projection",
                             "prefix": "forward with per-candidate prefix lengths "
                                       "(sorted U{0..L_r} per request)",
                             "backward": "backward pass (gradients of Z, W_Q, K/V for a "
                                         "N(0,1) dO)",
                             "backward_prefix": "backward pass with per-candidate prefix "
                                                "lengths (sorted U{0..L_r} per request)",
                             "codec": "forward over a coded memory, %.1f bits per coordinate"
                                      % args.codec_bits}[args.stage]},
        "timing": "HIP events on the launch stream around K back-to-back C-ABI calls with "
                  "pre-marshalled arguments (steps, then each kernel of a step alone); "
                  "%.0f ms untimed settle run before the W warm-up steps" % args.settle_ms,
        "roofline": roof, "cpu_baseline": cpu,
    }
    if others is not None:
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
