#!/usr/bin/env python3
"""Benchmark of the group-shared fixed fan-in tail layer on one MI355X.

A step is one fused training pass of the layer over one batch: forward
logits, BCE gradient against the 0/1 labels, weight gradient and feature
gradient (libhaste's haste_step), on the Amazon-3M-shaped workload
(L = 2,999,936 labels in groups of G = 32, F = 64, H = 768, B = 128, ~36
positives per sample; synthetic seeded inputs already resident in HBM).

Prints ONE JSON line.  Besides the required fields it carries
  roofline      the kernel with the larger share of the step (forward + BCE +
                dW, or the feature-gradient kernel) against HBM bandwidth:
                algorithmic bytes per launch over its average duration, from
                HIP events recorded around it on its stream (in a second pass
                of the same steps, so the timed region holds no events); `traffic` is the
                HBM bytes per launch that rocprofv3's FETCH_SIZE and WRITE_SIZE
                counters read for it, each scaled by what the same counter
                reads for a plain copy of known size (taken from the counter
                file under profiles/, and null when the kernel's sources have
                changed since those counters were taken);
  roofline_other the same figures for the other kernel;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same step;
  kernels_us    per-phase averages from the same events;
  extra         unfused calls and the G = 1 per-label baseline on the same
                shapes (speedups are time ratios at equal useful work).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tail-layer fwd+bwd samples/s and useful TFLOP/s (% bf16 MFMA peak), L=3M G=32"
CSRC = os.path.join(ROOT, "group_shared_fixed_amd", "csrc")
# sources each measured kernel is compiled from (for the counter file's validity)
KERNEL_SOURCES = {
    "k_group_fwd": ["k_fwd.hip", "common.hpp", "kernels.hpp"],
    "k_group_dh": ["k_dh.hip", "common.hpp", "kernels.hpp"],
}
COPY_BYTES = 1 << 30           # plain copy used to scale the byte counters

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (timing enabled) through libamdhip64."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev[i] = h
        self.n = n

    def block(self, i, k):
        """ctypes array view of events [i, i + k)."""
        return ctypes.cast(ctypes.addressof(self.ev) + i * ctypes.sizeof(ctypes.c_void_p),
                           ctypes.POINTER(ctypes.c_void_p))

    def record(self, i, stream):
        assert self.hip.hipEventRecord(self.ev[i], stream) == 0

    def ms(self, i, j):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[i], self.ev[j]) == 0
        return out.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.ev[i])


def source_sha256(kernel):
    import hashlib
    hsh = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()


def counter_file(workload):
    return os.path.join(ROOT, "profiles", f"hbm_counters_{workload}_step.json")


def read_counter_csv(path):
    """Average counter value per dispatch, by kernel base name, from a
    rocprofv3 counter_collection.csv."""
    import csv
    import re
    acc = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "").strip()
            key = (name, r["Counter_Name"])
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def ingest_counters(fetch_csv, write_csv, workload, commands):
    """Write the counter file from the FETCH_SIZE and WRITE_SIZE runs of
    `bench.py --counter-run` (KiB per dispatch)."""
    fetch, write = read_counter_csv(fetch_csv), read_counter_csv(write_csv)

    def pick(pred, counter, table):
        hits = [(v, k[0]) for k, v in table.items() if k[1] == counter and pred(k[0])]
        if not hits:
            raise SystemExit(f"no dispatch matching for {counter}")
        return max(hits)

    out = {"workload": workload, "unit": "KiB per dispatch", "commands": commands, "copy": {}, "kernels": {}}
    cf, cname = pick(lambda n: "elementwise" in n or "copy" in n.lower(), "FETCH_SIZE", fetch)
    cw, _ = pick(lambda n: n == cname, "WRITE_SIZE", write)
    out["copy"] = {"kernel": cname, "bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw}
    for kern in KERNEL_SOURCES:
        f, name = pick(lambda n, kern=kern: kern in n, "FETCH_SIZE", fetch)
        wv, _ = pick(lambda n, name=name: n == name, "WRITE_SIZE", write)
        out["kernels"][kern] = {"dispatch": name, "fetch_kib": f, "write_kib": wv,
                                "source_sha256": source_sha256(kern)}
    with open(counter_file(workload), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    log(f"[bench] wrote {counter_file(workload)}")


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the counter file, scaled by the
    copy calibration; None if absent or taken from other sources."""
    try:
        with open(counter_file(workload)) as fh:
            c = json.load(fh)
        k = c["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if k["source_sha256"] != source_sha256(kernel):
        return None
    cp = c["copy"]
    f_scale = cp["bytes"] / (cp["fetch_kib"] * 1024.0)
    w_scale = cp["bytes"] / (cp["write_kib"] * 1024.0)
    return int(round(1024.0 * (k["fetch_kib"] * f_scale + k["write_kib"] * w_scale)))


def bf16_dev(a, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def i32_dev(a, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def prepare_slots(hs, idx, W, G, args):
    """Puts each group's slots in the bank-balanced order (haste_order_slots,
    in place on idx and W's columns) unless --sorted-slots is given; the index
    sets themselves are unchanged.  Runs once, before any timing.  Returns the
    order's name for the JSON config."""
    if getattr(args, "sorted_slots", False):
        return "sorted (as drawn)"
    hs.order_slots(idx, W, G)
    import torch
    torch.cuda.synchronize()
    return "bank-balanced (haste_order_slots, applied once before timing)"


def time_call(fn, reps, stream_handle, ev):
    """Average ms of fn() over reps, from events on the call's stream."""
    fn()
    ev.record(0, stream_handle)
    for _ in range(reps):
        fn()
    ev.record(1, stream_handle)
    import torch
    torch.cuda.synchronize()
    return ev.ms(0, 1) / reps


def calibrate(dev, seconds=1.0):
    """What this GPU delivers to plain library kernels, measured in-process:
    an fp32 copy of 1 GiB (torch elementwise kernel: read + write bytes per
    second) and a dense bf16 GEMM of 8192^3 (torch.matmul, hipBLASLt).  They
    are the measured second denominators next to the spec peaks.  The GEMM
    runs for about `seconds`: a cold GPU otherwise spends its first few dozen
    steps below its working clock (measured: the on-chip-bound feature-
    gradient kernel 446 -> 397 us over its first 30 steps after an idle
    period, the HBM-bound forward 307 -> 298 us; 300 ms of copies did not
    remove it, one second of GEMMs did)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    e0.record()
    for _ in range(20):
        torch.mul(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_BYTES * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 0
    e0.record()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            torch.matmul(a, b, out=c)
        reps += 10
        torch.cuda.synchronize()
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_gbs": round(copy_gbs, 1), "bf16_gemm_tflops": round(gemm_tflops, 1),
            "copy": "torch.mul(src, 1.0, out=dst), fp32, 1 GiB in + 1 GiB out",
            "gemm": f"torch.matmul bf16 {n}^3 (hipBLASLt)"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# Run in a child process with OMP_NUM_THREADS=1: the oracle step on the
# 4k-label workload (whole) and on a slice of the 670K-shaped one.
_SINGLE_THREAD_SNIPPET = r"""
import json, sys, time
import numpy as np
sys.path.insert(0, ROOT)
from oracle import oracle as O
from synthetic import get_workload, make_inputs
res = {"threads": O.num_threads()}
for name, ngroups in (("tiny_4k", None), ("amazon670k_shaped", 1024)):
    w = get_workload(name)
    d = make_inputs(w, dZ=False)
    K = w.K if ngroups is None else ngroups
    lo, hi = 0, K * w.G
    rp, cols = [0], []
    for b in range(w.B):
        c = d["y_col"][d["y_rowptr"][b]:d["y_rowptr"][b + 1]]
        c = c[(c >= lo) & (c < hi)] - lo
        cols.append(c)
        rp.append(rp[-1] + c.size)
    t0 = time.perf_counter()
    O.oracle_step(d["h"], np.ascontiguousarray(d["idx"][:K]), np.ascontiguousarray(d["W"][:hi]),
                  np.array(rp, np.int32), np.concatenate(cols).astype(np.int32), 1.0 / w.B, w.G)
    el = time.perf_counter() - t0
    res[name] = {"groups": K, "of": w.K, "seconds": round(el, 3),
                 "seconds_per_step": round(el * w.K / K, 2), "samples_per_s": round(w.B / (el * w.K / K), 4)}
print(json.dumps(res))
"""


def cpu_single_thread(timeout=120):
    """Single-threaded oracle step timings (child process, OMP_NUM_THREADS=1)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = f"ROOT = {ROOT!r}\n" + _SINGLE_THREAD_SNIPPET
    try:
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=timeout)
        return json.loads(r.stdout.strip().splitlines()[-1]) if r.returncode == 0 else {"error": r.stderr[-300:]}
    except (subprocess.TimeoutExpired, ValueError, IndexError) as e:
        return {"error": str(e)[:300]}


def dense_point(w, d, dev, sh, ev, reps=10):
    """FLOPs-matched dense context: this library's fused step with H = F and
    every index set [0, F) (a dense bottleneck layer of the same useful
    FLOPs), and the three products of that dense layer as library GEMMs
    (torch.matmul on bf16, hipBLASLt; bf16 outputs, so they write half the
    bytes of the fp32 dW)."""
    import numpy as np
    import torch

    import group_shared_fixed_amd as hs
    B, K, G, F, L = w.B, w.K, w.G, w.F, w.L
    hF = bf16_dev(np.ascontiguousarray(d["h"][:, :F]), dev)
    W = bf16_dev(d["W"], dev)
    idxF = torch.arange(F, dtype=torch.int32, device=dev).repeat(K, 1).contiguous()
    rp, col = i32_dev(d["y_rowptr"], dev), i32_dev(d["y_col"], dev)
    out = {"dW": torch.empty(L, F, dtype=torch.float32, device=dev),
           "dh": torch.empty(B, F, dtype=torch.float32, device=dev), "Z": None, "loss": None}
    ws = torch.empty(hs.workspace_size("step", B, F, K, G, F, "det"), dtype=torch.uint8, device=dev)
    ours = 1e3 * time_call(lambda: hs.step(hF, idxF, W, rp, col, 1.0 / B, G, mode="det", out=out, workspace=ws),
                           reps, sh, ev)
    del out, ws, idxF
    WT = W.t().contiguous()                       # F x L
    dZ = bf16_dev(d["dZ"], dev) if "dZ" in d else torch.randn(B, L, device=dev).to(torch.bfloat16)
    dZT = dZ.t().contiguous()                     # L x B
    Z = torch.empty(B, L, dtype=torch.bfloat16, device=dev)
    dWl = torch.empty(L, F, dtype=torch.bfloat16, device=dev)
    dhl = torch.empty(B, F, dtype=torch.bfloat16, device=dev)
    t_f = 1e3 * time_call(lambda: torch.matmul(hF, WT, out=Z), reps, sh, ev)
    t_w = 1e3 * time_call(lambda: torch.matmul(dZT, hF, out=dWl), reps, sh, ev)
    t_h = 1e3 * time_call(lambda: torch.matmul(dZ, W, out=dhl), reps, sh, ev)
    del WT, dZT, Z, dWl, dhl, dZ, W, hF
    torch.cuda.empty_cache()
    return {"ours_step_dense_us": round(ours, 2),
            "library_gemms_us": {"fwd": round(t_f, 2), "dW": round(t_w, 2), "dh": round(t_h, 2),
                                 "sum": round(t_f + t_w + t_h, 2)},
            "what": f"haste_step at H = F = {F} with every I_k = [0, {F}); the dense layer's three products "
                    f"(B x F x L each) as torch.matmul bf16 GEMMs"}


def cpu_baseline(w, d, seconds):
    """The oracle (as is) on consecutive group slices, all batch rows, until
    `seconds` of wall time are spent; extrapolated to the whole step."""
    import numpy as np
    from oracle import oracle as O

    G, K, B = w.G, w.K, w.B
    s = 1.0 / B
    per = 4096
    done = 0
    t0 = time.perf_counter()
    while done < K and time.perf_counter() - t0 < seconds:
        k0, k1 = done, min(K, done + per)
        lo, hi = k0 * G, k1 * G
        rp = [0]
        cols = []
        for b in range(B):
            c = d["y_col"][d["y_rowptr"][b]:d["y_rowptr"][b + 1]]
            c = c[(c >= lo) & (c < hi)] - lo
            cols.append(c)
            rp.append(rp[-1] + c.size)
        O.oracle_step(d["h"], np.ascontiguousarray(d["idx"][k0:k1]), np.ascontiguousarray(d["W"][lo:hi]),
                      np.array(rp, np.int32), np.concatenate(cols).astype(np.int32), s, G)
        done = k1
    el = time.perf_counter() - t0
    t_full = el * K / done
    return {"value": round(B / t_full, 3), "unit": "samples/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"fp64 oracle step (fwd+BCE+dW+dh) on label groups [0, {done}) of {K}, all {B} samples; "
                      f"{el:.1f} s wall, extrapolated x{K / done:.2f} to the full step",
            "seconds_per_step": round(t_full, 3), "cpu_model": cpu_model()}


def sweep_g(args):
    """Per-G kernel times on the tail of the head-tail split (L = 2,910,848
    tail labels, F = 64, H = 768, B = 128, ~36 positives per sample): the
    fused step and the unfused calls for G = 16, 32, 64, and the per-label
    baseline (G = 1).  Same h and W for every G; index sets drawn per G."""
    import torch

    import group_shared_fixed_amd as hs
    from synthetic import get_workload, make_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    ev = HipEvents(8)
    reps = 10
    out = {"metric": "tail-layer kernel time per G (head-tail split, 3M)", "unit": "us", "n_gpus": 1,
           "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
           "config": {"workload": "ht3m_tail_shaped", "L": 2910848, "F": 64, "H": 768, "B": 128,
                      "dh_mode": args.mode}, "per_G": {}}
    for G in (16, 32, 64, 1):
        w = get_workload("ht3m_tail_shaped", G=max(G, 16))
        log(f"[sweep] G={G}: generating")
        d = make_inputs(w, dZ=True, idx1=(G == 1))
        B, H, F, L = w.B, w.H, w.F, w.L
        K = L // max(G, 1)
        h, W, dZ = bf16_dev(d["h"], dev), bf16_dev(d["W"], dev), bf16_dev(d["dZ"], dev)
        rp, col = i32_dev(d["y_rowptr"], dev), i32_dev(d["y_col"], dev)
        Z = torch.empty(B, L, dtype=torch.float32, device=dev)
        dW = torch.empty(L, F, dtype=torch.float32, device=dev)
        dh = torch.empty(B, H, dtype=torch.float32, device=dev)
        r = {}
        if G == 1:
            idx1 = i32_dev(d["idx1"], dev)
            ws = torch.empty(max(256, hs.workspace_size("fixed_bwd_h", B, H, L, 1, F, "det")),
                             dtype=torch.uint8, device=dev)
            r["fwd_us"] = 1e3 * time_call(lambda: hs.fixed_fwd(h, idx1, W, Z=Z, workspace=ws), reps, sh, ev)
            r["bwd_w_us"] = 1e3 * time_call(lambda: hs.fixed_bwd_w(h, idx1, dZ, dW=dW, workspace=ws), reps, sh, ev)
            r["bwd_h_us"] = 1e3 * time_call(lambda: hs.fixed_bwd_h(dZ, idx1, W, H, mode=args.mode, dh=dh,
                                                                   workspace=ws), reps, sh, ev)
        else:
            idx = i32_dev(d["idx"], dev)
            r["slot_order"] = prepare_slots(hs, idx, W, G, args)
            ws = torch.empty(max(256, hs.workspace_size("step", B, H, K, G, F, "det")), dtype=torch.uint8,
                             device=dev)
            o = {"dW": dW, "dh": dh, "Z": None, "loss": None}
            r["step_us"] = 1e3 * time_call(lambda: hs.step(h, idx, W, rp, col, 1.0 / B, G, mode=args.mode, out=o,
                                                           workspace=ws), reps, sh, ev)
            r["fwd_us"] = 1e3 * time_call(lambda: hs.fwd(h, idx, W, G, Z=Z, workspace=ws), reps, sh, ev)
            r["bwd_w_us"] = 1e3 * time_call(lambda: hs.bwd_w(h, idx, dZ, G, dW=dW, workspace=ws), reps, sh, ev)
            r["bwd_h_us"] = 1e3 * time_call(lambda: hs.bwd_h(dZ, idx, W, G, H, mode=args.mode, dh=dh,
                                                             workspace=ws), reps, sh, ev)
            r["step_samples_per_s"] = round(B / (r["step_us"] * 1e-6), 1)
        out["per_G"][str(G)] = {k: round(v, 2) if isinstance(v, float) else v for k, v in r.items()}
        log(f"[sweep] G={G}: {out['per_G'][str(G)]}")
        del Z, dW, dh, d
        torch.cuda.empty_cache()
    base = out["per_G"]["1"]
    for G in ("16", "32", "64"):
        g = out["per_G"][G]
        g["speedup_fwd_vs_G1"] = round(base["fwd_us"] / g["fwd_us"], 2)
        g["speedup_bwd_vs_G1"] = round((base["bwd_w_us"] + base["bwd_h_us"]) / (g["bwd_w_us"] + g["bwd_h_us"]), 2)
    ev.close()
    line = json.dumps(out)
    print(line, flush=True)
    if args.report:
        with open(args.report, "w") as fh:
            fh.write(line + "\n")


def joint_bench(args):
    """The joint head + tail step of the head-tail split at 3M (haste_joint_step):
    89,088 dense-head labels and 2,910,848 tail labels (G = 32, F = 64),
    H = 768, B = 128, ~36 positives per sample drawn over the full label
    space and split.  One JSON line: joint samples/s, the two branches timed
    alone, the head pass against HBM bandwidth, and the oracle on the CPU."""
    import numpy as np
    import torch

    import group_shared_fixed_amd as hs
    from synthetic import get_workload, make_inputs

    w = get_workload("ht3m_tail_shaped")
    B, H, K, G, F, L, Lh = w.B, w.H, w.K, w.G, w.F, w.L, w.head_labels
    dev = torch.device("cuda:0")
    log(f"[joint] generating {w.name}: tail L={L} G={G} F={F}, head {Lh} x {H}, B={B}")
    d = make_inputs(w, dZ=False, w_head=True)
    h, idx, Wt, Wh = (bf16_dev(d["h"], dev), i32_dev(d["idx"], dev), bf16_dev(d["W"], dev),
                      bf16_dev(d["W_head"], dev))
    yt = (i32_dev(d["y_rowptr"], dev), i32_dev(d["y_col"], dev))
    yh = (i32_dev(d["yh_rowptr"], dev), i32_dev(d["yh_col"], dev))
    slot_order = prepare_slots(hs, idx, Wt, G, args)
    s = 1.0 / B
    out = {"dW_tail": torch.empty(L, F, dtype=torch.float32, device=dev),
           "dW_head": torch.empty(Lh, H, dtype=torch.float32, device=dev),
           "dh": torch.empty(B, H, dtype=torch.float32, device=dev), "loss": None}
    ws = torch.empty(hs.joint_workspace_size(B, H, K, G, F, Lh, args.mode), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    ev = HipEvents(4)

    def run():
        hs.joint_step(h, idx, Wt, *yt, Wh, *yh, s, s, G, mode=args.mode, out=out, workspace=ws)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / args.steps
    o_t = {"dW": out["dW_tail"], "dh": out["dh"], "Z": None, "loss": None}
    o_h = {"dW": out["dW_head"], "dh": out["dh"], "Z": None, "loss": None}
    reps = max(10, args.steps // 2)
    tail_us = 1e3 * time_call(lambda: hs.step(h, idx, Wt, *yt, s, G, mode=args.mode, out=o_t, workspace=ws),
                              reps, sh, ev)
    head_us = 1e3 * time_call(lambda: hs.head_step(h, Wh, *yh, s, out=o_h, workspace=ws), reps, sh, ev)
    log(f"[joint] step {ms_step:.3f} ms; tail alone {tail_us:.1f} us, head alone {head_us:.1f} us")
    nnz_h = int(d["yh_rowptr"][-1])
    # head pass, every compulsory tensor once: W_head, h, head labels in; dW_head, dh out
    head_bytes = Lh * H * 2 + B * H * 2 + (B + 1) * 4 + nnz_h * 4 + Lh * H * 4 + B * H * 4
    head_flops = 3 * 2 * B * Lh * H
    tail_flops = 6 * B * L * F
    ach = head_bytes / (head_us * 1e-6) / 1e9
    res = {
        "metric": "joint head+tail step samples/s (head-tail split, 3M labels)",
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ht3m_joint_shaped", "L_head": Lh, "L_tail": L, "G": G, "K": K, "F": F, "H": H,
                   "B": B, "positives_per_sample": w.m, "dh_mode": args.mode, "slot_order": slot_order,
                   "step": "haste_joint_step: tail haste_step, then the dense head (logits + BCE, dW and dh kernels)"},
        "useful_tflops": round((head_flops + tail_flops) / (ms_step * 1e-3) / 1e12, 2),
        "branches_us": {"tail_step": round(tail_us, 2), "head_step": round(head_us, 2)},
        "roofline_head": {"kernel": "head pass (logits + BCE, dW, dh, dh sum)", "bound": "hbm",
                          "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": head_bytes,
                          "avg_us": round(head_us, 2), "head_tflops": round(head_flops / (head_us * 1e-6) / 1e12, 2)},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        log("[joint] timing the CPU oracle")
        cb = cpu_baseline(w, d, args.cpu_seconds)
        t0 = time.perf_counter()
        O.oracle_head_step(d["h"], d["W_head"], d["yh_rowptr"], d["yh_col"], s)
        t_head = time.perf_counter() - t0
        t_all = cb["seconds_per_step"] + t_head
        res["cpu_baseline"] = {"value": round(B / t_all, 3), "unit": "samples/s", "cores": cb["cores"],
                               "kind": "oracle",
                               "sample": cb["sample"] + f"; plus the whole fp64 head pass ({t_head:.2f} s)",
                               "seconds_per_step": round(t_all, 3)}
    ev.close()
    line = json.dumps(res)
    print(line, flush=True)
    if args.report:
        with open(args.report, "w") as fh:
            fh.write(line + "\n")


def w8_bench(args):
    """The fused step with FP8 (E4M3) weights (haste_step_w8) on the
    Amazon-3M shape, next to the bf16 step on the same (dequantized) weights
    in the same process.  One JSON line: samples/s of both, per-kernel event
    averages, the dominant kernel against HBM bandwidth with the FP8
    algorithmic bytes, and the quantizer's time."""
    import numpy as np
    import torch

    import group_shared_fixed_amd as hs
    from synthetic import get_workload, make_inputs

    w = get_workload(args.workload)
    B, H, K, G, F, L = w.B, w.H, w.K, w.G, w.F, w.L
    dev = torch.device("cuda:0")
    log(f"[w8] generating {w.name}: L={L} G={G} K={K} F={F} H={H} B={B}")
    d = make_inputs(w, dZ=False)
    h, idx, W = bf16_dev(d["h"], dev), i32_dev(d["idx"], dev), bf16_dev(d["W"], dev)
    rp, col = i32_dev(d["y_rowptr"], dev), i32_dev(d["y_col"], dev)
    slot_order = prepare_slots(hs, idx, W, G, args)
    W8, wexp = hs.quantize_w8(W, G)
    # the bf16 weights the FP8 step computes with, for the side-by-side step
    Wq = torch.empty_like(W)
    Wq.view(torch.int16).copy_(torch.from_numpy(dequant_host(W8.cpu().numpy(), wexp.cpu().numpy(), G)
                                                ).view(torch.int16).to(dev))
    s = 1.0 / B
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    out = {"dW": torch.empty(L, F, dtype=torch.float32, device=dev),
           "dh": torch.empty(B, H, dtype=torch.float32, device=dev), "Z": None, "loss": None}
    ws = torch.empty(max(256, hs.workspace_size("step", B, H, K, G, F, args.mode)), dtype=torch.uint8, device=dev)
    ev = HipEvents(5 * args.steps + 2)

    def timed(fn):
        for _ in range(args.warmup):
            fn(None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn(None)
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t0) / args.steps
        for i in range(args.steps):
            fn(ev.block(5 * i, 5))
        torch.cuda.synchronize()

        def avg(a, b):
            return 1e3 * sum(ev.ms(5 * i + a, 5 * i + b) for i in range(args.steps)) / args.steps

        return ms, {"fwd_bce_dw_us": round(avg(1, 2), 2), "dh_us": round(avg(2, 3), 2),
                    "dh_reduce_us": round(avg(3, 4), 2)}

    ms8, ph8 = timed(lambda e: hs.step_w8(h, idx, W8, wexp, rp, col, s, G, mode=args.mode, out=out, workspace=ws,
                                          events=e))
    ms16, ph16 = timed(lambda e: hs.step(h, idx, Wq, rp, col, s, G, mode=args.mode, out=out, workspace=ws,
                                         events=e))
    q_ms = time_call(lambda: hs.quantize_w8(W, G, W8=W8, wexp=wexp), 20, sh, ev)
    log(f"[w8] fp8-weight step {ms8:.3f} ms {ph8}; bf16 step {ms16:.3f} ms {ph16}; quantize {1e3 * q_ms:.1f} us")
    nnz = int(d["y_rowptr"][-1])
    lab = (B + 1) * 4 + nnz * 4
    bytes_a = L * F * 1 + K * 4 + K * F * 4 + B * H * 2 + lab + L * F * 4
    bytes_b = L * F * 1 + K * 4 + K * F * 4 + B * H * 2 + lab + B * H * 4
    dom_us, dom_b, dom_k = ((ph8["dh_us"], bytes_b, "k_group_dh32<..., FP8 weights> (feature gradient)")
                            if ph8["dh_us"] >= ph8["fwd_bce_dw_us"] else
                            (ph8["fwd_bce_dw_us"], bytes_a, "k_group_fwd<..., FP8 weights> (forward + BCE + dW)"))
    ach = dom_b / (dom_us * 1e-6) / 1e9
    res = {
        "metric": "tail-layer fwd+bwd samples/s with FP8 (E4M3) weights, L=3M G=32",
        "value": round(B / (ms8 * 1e-3), 1), "unit": "samples/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms8, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 compute, fp8 e4m3 weights", "data": "synthetic",
        "config": {"workload": w.name, "L": L, "G": G, "K": K, "F": F, "H": H, "B": B, "dh_mode": args.mode,
                   "slot_order": slot_order,
                   "step": "haste_step_w8: fused forward + BCE + dW + dh from E4M3 weights with group exponents"},
        "kernels_us": ph8,
        "bf16_step": {"ms_per_step": round(ms16, 4), "samples_per_s": round(B / (ms16 * 1e-3), 1),
                      "kernels_us": ph16},
        "speedup_vs_bf16_step": round(ms16 / ms8, 3),
        "quantize_us": round(1e3 * q_ms, 2),
        "roofline": {"kernel": dom_k, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes": dom_b, "avg_us": round(dom_us, 2)},
    }
    ev.close()
    line = json.dumps(res)
    print(line, flush=True)
    if args.report:
        with open(args.report, "w") as fh:
            fh.write(line + "\n")


def dequant_host(W8, wexp, G):
    """bf16 bits of decode(code) * 2^wexp: the E4M3 format's definition on the host
    (used to build the bf16 step that runs beside the FP8 one)."""
    import numpy as np
    c = W8.astype(np.int64)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.ldexp(1.0, e - 10))
    val = np.where(c & 0x80, -mag, mag) * np.ldexp(1.0, np.repeat(wexp.astype(np.int64), G))[:, None]
    return (val.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def grouping_bench(args):
    """Semantic label grouping at the Amazon-3M label count: L = 2,999,936
    synthetic unit embeddings (H = 768, 4,096 topics), C = L / (4 G) =
    23,437 clusters for G = 32; k-means init, --km-iters mini-batch steps of
    65,536 labels, the full assignment and the greedy groups.  One JSON line:
    the whole pipeline's seconds, the phases (HIP events), the assignment
    products against the bf16 matrix-core peak, and the oracle on the CPU."""
    import numpy as np
    import torch

    import group_shared_fixed_amd as hs
    from synthetic import kmeans_draws, label_embeddings

    L, H, G = 2_999_936, 768, 32
    C, nb, iters = L // (4 * G), 65536, args.km_iters
    dev = torch.device("cuda:0")
    log(f"[grouping] generating {L} embeddings (H = {H}), C = {C}, {iters} mini-batch steps of {nb}")
    E = label_embeddings(L, H, 4096, 0.6, 97)
    init, batches = kmeans_draws(L, C, nb, iters, 97)
    Ed = bf16_dev(E, dev)
    init_d = i32_dev(init, dev)
    batch_d = [i32_dev(b, dev) for b in batches]
    ws_a = torch.empty(max(hs.binding.lib().haste_kmeans_assign_workspace_size(L, C, H, 0),
                           hs.binding.lib().haste_kmeans_assign_workspace_size(nb, C, H, 1)), dtype=torch.uint8,
                       device=dev)
    ws_u = torch.empty(hs.binding.lib().haste_kmeans_update_workspace_size(nb, C), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(hs.binding.lib().haste_group_workspace_size(L, C), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    ev = HipEvents(2 * iters + 8)

    def pipeline(mark):
        mark(0)
        Mc, Mb, v = hs.kmeans_init(Ed, init_d)
        for i, b in enumerate(batch_d):
            a_b, _ = hs.kmeans_assign(Ed, Mb, rows=b, workspace=ws_a)
            mark(1 + 2 * i)
            hs.kmeans_update(Ed, b, a_b, Mc, Mb, v, workspace=ws_u)
            mark(2 + 2 * i)
        a, _ = hs.kmeans_assign(Ed, Mb, workspace=ws_a)
        mark(2 * iters + 1)
        perm = hs.group_greedy(Ed, a, C, G, workspace=ws_g)
        mark(2 * iters + 2)
        return perm

    pipeline(lambda i: None)                       # warm-up (library code objects, caches)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pipeline(lambda i: None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pipeline(lambda i: ev.record(i, sh))
    torch.cuda.synchronize()
    step_assign = sum(ev.ms(2 * i, 2 * i + 1) for i in range(iters)) / iters
    step_update = sum(ev.ms(2 * i + 1, 2 * i + 2) for i in range(iters)) / iters
    full_assign = ev.ms(2 * iters, 2 * iters + 1)
    greedy = ev.ms(2 * iters + 1, 2 * iters + 2)
    flops_full = 2.0 * L * C * H
    tf = flops_full / (full_assign * 1e-3) / 1e12
    log(f"[grouping] pipeline {wall:.3f} s; step assign {step_assign:.2f} ms, update {step_update:.3f} ms; "
        f"full assign {full_assign:.1f} ms ({tf:.0f} TFLOP/s); greedy {greedy:.1f} ms")
    res = {
        "metric": "label grouping time (mini-batch spherical k-means + greedy groups), 3M labels",
        "value": round(wall, 4), "unit": "s", "n_gpus": 1, "steps": 1, "warmup": 1,
        "ms_per_step": round(1e3 * wall, 2), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "grouping_3m", "L": L, "H": H, "G": G, "C": C, "minibatch": nb, "iters": iters,
                   "step": "kmeans_init + iters x (assign batch + update) + full assign + group_greedy"},
        "phases_ms": {"minibatch_assign": round(step_assign, 3), "minibatch_update": round(step_update, 3),
                      "full_assign": round(full_assign, 2), "greedy": round(greedy, 2)},
        "roofline": {"kernel": "full assignment (k_assign: fused matrix-core scores + arg-max)",
                     "bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None, "algorithmic_flops": flops_full,
                     "avg_us": round(1e3 * full_assign, 1)},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        log("[grouping] timing the CPU oracle")
        M = np.ascontiguousarray(E[init])
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < args.cpu_seconds / 2 and done < L:
            O.oracle_kmeans_assign(np.ascontiguousarray(E[done:done + 4096]), M)
            done += 4096
        t_assign = (time.perf_counter() - t0) / done                 # s per label
        t0 = time.perf_counter()
        n_lab = 0
        for c in range(C):
            if time.perf_counter() - t0 > args.cpu_seconds / 2:
                break
            sub = np.ascontiguousarray(E[c * 128:(c + 1) * 128])
            O.oracle_group_greedy(sub, np.zeros(128, np.int32), 1, G)
            n_lab += 128
        t_greedy = (time.perf_counter() - t0) / max(n_lab, 1)
        t_all = (L + iters * nb) * t_assign + L * t_greedy
        res["cpu_baseline"] = {"value": round(t_all, 1), "unit": "s", "cores": O.num_threads(), "kind": "oracle",
                               "sample": f"oracle assignment of {done} labels against all {C} centres and greedy "
                                         f"groups of {n_lab} labels in clusters of 128, extrapolated to the "
                                         f"pipeline ({L} + {iters} x {nb} assignments, {L} labels grouped)"}
    ev.close()
    line = json.dumps(res)
    print(line, flush=True)
    if args.report:
        with open(args.report, "w") as fh:
            fh.write(line + "\n")


def rewire_bench(args):
    """Group-level rewiring (haste_rewire) on the Amazon-3M shape: K =
    93,748 groups of G = 32, F = 64, H = 768, B = 128, dZ ~ N(0, 1) bf16,
    --n-swap slots per group (default 16).  One JSON line: calls/s, the
    score kernel against the bf16 matrix-core peak and the selection kernel
    against HBM bandwidth (HIP events on the launch stream), and the oracle
    on the CPU."""
    import numpy as np
    import torch

    import group_shared_fixed_amd as hs
    from synthetic import get_workload, make_inputs

    w = get_workload("amazon3m_shaped")
    B, H, K, G, F, L = w.B, w.H, w.K, w.G, w.F, w.L
    n = args.n_swap
    dev = torch.device("cuda:0")
    log(f"[rewire] generating {w.name}: L={L} G={G} K={K} F={F} H={H} B={B}, n_swap={n}")
    d = make_inputs(w, dZ=True, labels=False)
    h, dZ, idx, W = bf16_dev(d["h"], dev), bf16_dev(d["dZ"], dev), i32_dev(d["idx"], dev), bf16_dev(d["W"], dev)
    idx_o, W_o = torch.empty_like(idx), torch.empty_like(W)
    ws = torch.empty(hs.rewire_workspace_size(B, H, K, G, F), dtype=torch.uint8, device=dev)
    ev = HipEvents(4 * args.steps + 2)

    def run(i=None):
        hs.rewire(h, dZ, idx, W, G, n, idx_out=idx_o, W_out=W_o, workspace=ws,
                  events=None if i is None else ev.block(4 * i, 4))

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()

    def avg(a, b):
        return sum(ev.ms(4 * i + a, 4 * i + b) for i in range(args.steps)) / args.steps

    score_us, select_us = 1e3 * avg(1, 2), 1e3 * avg(2, 3)
    flops = 2 * B * L * H                       # the dense gradient dZ^T h
    score_bytes = B * L * 2 + B * H * 2 + K * H * 4
    select_bytes = K * H * 4 + 2 * (L * F * 2 + K * F * 4)
    tf = flops / (score_us * 1e-6) / 1e12
    sel_gbs = select_bytes / (select_us * 1e-6) / 1e9
    log(f"[rewire] {ms:.3f} ms per call; score {score_us:.1f} us ({tf:.0f} TFLOP/s), select {select_us:.1f} us")
    res = {
        "metric": "group-level rewiring calls/s (haste_rewire, Amazon-3M shape)",
        "value": round(1e3 / ms, 2), "unit": "calls/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "L": L, "G": G, "K": K, "F": F, "H": H, "B": B, "n_swap": n,
                   "step": "haste_rewire: grow scores (dense dZ^T h on matrix cores) + per-group selection"},
        "kernels_us": {"prep_us": round(1e3 * avg(0, 1), 2), "score_us": round(score_us, 2),
                       "select_us": round(select_us, 2)},
        "roofline": {"kernel": "k_rewire_score (dense gradient, |.| summed per group)", "bound": "mfma",
                     "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None, "algorithmic_flops": flops,
                     "algorithmic_bytes": score_bytes, "avg_us": round(score_us, 2)},
        "roofline_other": {"kernel": "k_rewire_select", "bound": "hbm", "achieved": round(sel_gbs, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(sel_gbs / HBM_PEAK_GBS, 4),
                           "traffic": None, "algorithmic_bytes": select_bytes, "avg_us": round(select_us, 2)},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        log("[rewire] timing the CPU oracle")
        per, done = 256, 0
        t0 = time.perf_counter()
        while done < K and time.perf_counter() - t0 < args.cpu_seconds:
            k0, k1 = done, min(K, done + per)
            idx_s = np.ascontiguousarray(d["idx"][k0:k1])
            W_s = np.ascontiguousarray(d["W"][k0 * G:k1 * G])
            dZ_s = np.ascontiguousarray(d["dZ"][:, k0 * G:k1 * G])
            O.oracle_rewire(d["h"], dZ_s, idx_s, W_s, n, G)
            done = k1
        el = time.perf_counter() - t0
        t_full = el * K / done
        res["cpu_baseline"] = {"value": round(1.0 / t_full, 5), "unit": "calls/s", "cores": O.num_threads(),
                               "kind": "oracle",
                               "sample": f"oracle rewiring (numpy fp64 scores, Python selection) on groups "
                                         f"[0, {done}) of {K}; {el:.1f} s wall, extrapolated x{K / done:.1f}",
                               "seconds_per_call": round(t_full, 2)}
    ev.close()
    line = json.dumps(res)
    print(line, flush=True)
    if args.report:
        with open(args.report, "w") as fh:
            fh.write(line + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="amazon3m_shaped")
    ap.add_argument("--mode", default="det", choices=["atomic", "det"],
                    help="dh reduction (deterministic is the default: bitwise reproducible and, with the "
                         "split-K partials written once and summed in order, faster than fp32 atomics)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip unfused calls and the G=1 baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the FLOPs-matched dense point")
    ap.add_argument("--no-calibrate", action="store_true",
                    help="skip the copy / GEMM calibration before the warm-up steps")
    ap.add_argument("--report", default=None, help="also write the JSON line to this file")
    ap.add_argument("--counter-run", action="store_true",
                    help="short run for rocprofv3 --pmc: a few steps plus a plain 1 GiB copy, no JSON line")
    ap.add_argument("--ingest", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the counter file under profiles/ from the two --counter-run counter CSVs")
    ap.add_argument("--commands", default="", help="with --ingest: the profiling commands, recorded in the file")
    ap.add_argument("--sweep-g", action="store_true",
                    help="tail of the head-tail split at 3M (2,910,848 labels): per-G timings for G in "
                         "{16, 32, 64} and the G = 1 baseline, one JSON line")
    ap.add_argument("--joint", action="store_true",
                    help="joint head + tail step of the 3M head-tail split (haste_joint_step), one JSON line")
    ap.add_argument("--rewire", action="store_true",
                    help="group-level rewiring (haste_rewire) on the Amazon-3M shape, one JSON line")
    ap.add_argument("--n-swap", type=int, default=16, help="with --rewire: slots replaced per group")
    ap.add_argument("--grouping", action="store_true",
                    help="semantic label grouping (k-means + greedy groups) at 3M labels, one JSON line")
    ap.add_argument("--km-iters", type=int, default=20, help="with --grouping: mini-batch k-means steps")
    ap.add_argument("--sorted-slots", action="store_true",
                    help="keep each group's slots in the drawn (sorted) order instead of the bank-balanced order")
    ap.add_argument("--w8", action="store_true",
                    help="the fused step with FP8 (E4M3) weights next to the bf16 step, one JSON line")
    args = ap.parse_args()

    if args.ingest:
        ingest_counters(args.ingest[0], args.ingest[1], args.workload, args.commands)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer is built and measured on a single MI355X; "
              "multi-GPU runs are not supported (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    if args.sweep_g:
        return sweep_g(args)
    if args.joint:
        return joint_bench(args)
    if args.rewire:
        return rewire_bench(args)
    if args.w8:
        return w8_bench(args)
    if args.grouping:
        return grouping_bench(args)

    import numpy as np
    import torch

    import group_shared_fixed_amd as hs
    from synthetic import get_workload, make_inputs

    w = get_workload(args.workload)
    B, H, K, G, F, L = w.B, w.H, w.K, w.G, w.F, w.L
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}: L={L} G={G} K={K} F={F} H={H} B={B}")
    t0 = time.time()
    d = make_inputs(w, dZ=not args.no_extra, idx1=not args.no_extra)
    log(f"[bench] inputs ready in {time.time() - t0:.1f} s")

    h, idx, W = bf16_dev(d["h"], dev), i32_dev(d["idx"], dev), bf16_dev(d["W"], dev)
    rp, col = i32_dev(d["y_rowptr"], dev), i32_dev(d["y_col"], dev)
    slot_order = prepare_slots(hs, idx, W, G, args)
    s = 1.0 / B
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    out = {"dW": torch.empty(L, F, dtype=torch.float32, device=dev),
           "dh": torch.empty(B, H, dtype=torch.float32, device=dev), "Z": None, "loss": None}
    ws = torch.empty(max(256, hs.workspace_size("step", B, H, K, G, F, args.mode)), dtype=torch.uint8, device=dev)

    if args.counter_run:
        for _ in range(3):
            hs.step(h, idx, W, rp, col, s, G, mode=args.mode, out=out, workspace=ws)
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("[bench] counter run done (3 steps, 2 copies of 1 GiB)")
        return

    machine = None
    if not args.no_calibrate:
        log("[bench] calibrating (copy, dense bf16 GEMM)")
        machine = calibrate(dev)
        log(f"[bench] copy {machine['copy_gbs']} GB/s, bf16 GEMM {machine['bf16_gemm_tflops']} TFLOP/s")

    nev = 5 * args.steps
    ev = HipEvents(nev + 2)

    def run(i=None):
        hs.step(h, idx, W, rp, col, s, G, mode=args.mode, out=out, workspace=ws,
                events=None if i is None else ev.block(5 * i, 5))

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # timed region: plain steps, no events inside
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    # phase breakdown: the same steps again with HIP events between the kernels
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()

    def avg(a, b):
        return sum(ev.ms(5 * i + a, 5 * i + b) for i in range(args.steps)) / args.steps

    ph = {"prep_us": 1e3 * avg(0, 1), "fwd_bce_dw_us": 1e3 * avg(1, 2), "dh_us": 1e3 * avg(2, 3),
          "dh_reduce_us": 1e3 * avg(3, 4), "step_events_us": 1e3 * avg(0, 4)}
    nnz = int(d["y_rowptr"][-1])
    labels_bytes = (B + 1) * 4 + nnz * 4
    # algorithmic bytes per launch: every input read once from HBM, every output written once
    # forward + BCE + dW: W, idx, h, labels in; dW out
    bytes_a = L * F * 2 + K * F * 4 + B * H * 2 + labels_bytes + L * F * 4
    # feature gradient: W, idx, h, labels in; dh out
    bytes_b = L * F * 2 + K * F * 4 + B * H * 2 + labels_bytes + B * H * 4
    flops_step = 6 * B * L * F
    useful_tflops = flops_step / (ms_step * 1e-3) / 1e12
    step_bytes = bytes_a + B * H * 4

    def roof(kernel, label, nbytes, us):
        ach = nbytes / (us * 1e-6) / 1e9
        r = {"kernel": label, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name, kernel),
             "algorithmic_bytes": nbytes, "avg_us": round(us, 2)}
        if machine:
            r["peak_measured"] = machine["copy_gbs"]
            r["frac_measured"] = round(ach / machine["copy_gbs"], 4)
        return r

    ra = roof("k_group_fwd", "k_group_fwd<STEP_DW> (forward + BCE + dW)", bytes_a, ph["fwd_bce_dw_us"])
    rb = roof("k_group_dh", "k_group_dh32 / k_group_dh, from labels (feature gradient, logits recomputed)", bytes_b,
              ph["dh_us"])
    dom, other = (rb, ra) if ph["dh_us"] >= ph["fwd_bce_dw_us"] else (ra, rb)
    res = {
        "metric": METRIC,
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "L": L, "G": G, "K": K, "F": F, "H": H, "B": B,
                   "positives_per_sample": w.m, "dh_mode": args.mode, "slot_order": slot_order,
                   "step": "haste_step: fused forward + BCE gradient + dW + dh"},
        "useful_tflops": round(useful_tflops, 2),
        "pct_bf16_peak": round(100 * useful_tflops / BF16_PEAK_TFLOPS, 2),
        "step_hbm_floor_us": round(step_bytes / HBM_PEAK_GBS / 1e3, 1),
        "roofline": dom,
        "roofline_other": other,
        "kernels_us": {k: round(v, 2) for k, v in ph.items()},
    }
    if machine:
        res["machine"] = machine
        res["pct_measured_gemm"] = round(100 * useful_tflops / machine["bf16_gemm_tflops"], 2)
    log(f"[bench] step {ms_step:.3f} ms  phases {res['kernels_us']}")

    if not args.no_extra:
        extra = {}
        dZ = bf16_dev(d["dZ"], dev)
        idx1 = i32_dev(d["idx1"], dev)
        Z = torch.empty(B, L, dtype=torch.float32, device=dev)
        dW = torch.empty(L, F, dtype=torch.float32, device=dev)
        dh = torch.empty(B, H, dtype=torch.float32, device=dev)
        wsx = torch.empty(max(256, hs.workspace_size("step", B, H, K, G, F, "det")), dtype=torch.uint8, device=dev)
        out16 = {"dW": torch.empty(L, F, dtype=torch.bfloat16, device=dev), "dh": dh, "Z": None, "loss": None}
        reps = 10
        calls = {
            "fwd": lambda: hs.fwd(h, idx, W, G, Z=Z, workspace=wsx),
            "bwd_w": lambda: hs.bwd_w(h, idx, dZ, G, dW=dW, workspace=wsx),
            "bwd_h_atomic": lambda: hs.bwd_h(dZ, idx, W, G, H, mode="atomic", dh=dh, workspace=wsx),
            "bwd_h_det": lambda: hs.bwd_h(dZ, idx, W, G, H, mode="det", dh=dh, workspace=wsx),
            "step_other_mode": lambda: hs.step(h, idx, W, rp, col, s, G,
                                               mode="det" if args.mode == "atomic" else "atomic",
                                               out=out, workspace=wsx),
            # the same step with dW stored as bf16 (haste_step_bf16dw): half the dW write
            "step_bf16_dw": lambda: hs.step(h, idx, W, rp, col, s, G, mode=args.mode, out=out16, workspace=wsx,
                                            dw_bf16=True),
            "fixed_fwd": lambda: hs.fixed_fwd(h, idx1, W, Z=Z, workspace=wsx),
            "fixed_bwd_w": lambda: hs.fixed_bwd_w(h, idx1, dZ, dW=dW, workspace=wsx),
            "fixed_bwd_h_atomic": lambda: hs.fixed_bwd_h(dZ, idx1, W, H, mode="atomic", dh=dh, workspace=wsx),
        }
        for name, fn in calls.items():
            extra[name + "_us"] = round(1e3 * time_call(fn, reps, sh, ev), 2)
            log(f"[bench] {name}: {extra[name + '_us']} us")
        t_fwd_bce = time_call(lambda: hs.fwd_bce(h, idx, W, rp, col, s, G, workspace=wsx), reps, sh, ev)
        extra["fwd_bce_us"] = round(1e3 * t_fwd_bce, 2)
        unf = extra["fwd_bce_us"] + extra["bwd_w_us"] + extra["bwd_h_atomic_us"]
        extra["unfused_step_us"] = round(unf, 2)
        extra["step_bf16_dw_samples_per_s"] = round(B / (extra["step_bf16_dw_us"] * 1e-6), 1)
        for i in range(args.steps):
            hs.step(h, idx, W, rp, col, s, G, mode=args.mode, out=out16, workspace=wsx, dw_bf16=True,
                    events=ev.block(5 * i, 5))
        torch.cuda.synchronize()
        extra["step_bf16_dw_kernels_us"] = {"fwd_bce_dw_us": round(1e3 * avg(1, 2), 2),
                                            "dh_us": round(1e3 * avg(2, 3), 2)}
        log(f"[bench] step_bf16_dw phases: {extra['step_bf16_dw_kernels_us']}")
        extra["speedup_fwd_vs_G1"] = round(extra["fixed_fwd_us"] / extra["fwd_us"], 2)
        extra["speedup_bwd_vs_G1"] = round((extra["fixed_bwd_w_us"] + extra["fixed_bwd_h_atomic_us"]) /
                                           (extra["bwd_w_us"] + extra["bwd_h_atomic_us"]), 2)
        # every call against its own HBM floor (compulsory bytes once at 8 TB/s)
        floors = {
            "fwd": L * F * 2 + K * F * 4 + B * H * 2 + B * L * 4,
            "bwd_w": B * L * 2 + K * F * 4 + B * H * 2 + L * F * 4,
            "bwd_h_atomic": B * L * 2 + L * F * 2 + K * F * 4 + B * H * 4,
            "bwd_h_det": B * L * 2 + L * F * 2 + K * F * 4 + B * H * 4,
            "fixed_fwd": L * F * 4 + L * F * 2 + B * H * 2 + B * L * 4,
            "fixed_bwd_w": L * F * 4 + B * L * 2 + B * H * 2 + L * F * 4,
            "fixed_bwd_h_atomic": L * F * 4 + L * F * 2 + B * L * 2 + B * H * 4,
        }
        for name, nbytes in floors.items():
            extra[name + "_hbm_frac"] = round(nbytes / (extra[name + "_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        res["extra"] = extra
        del Z, dW, dh, dZ, idx1, out16
        torch.cuda.empty_cache()
        if not args.no_dense:
            log("[bench] FLOPs-matched dense point")
            res["dense_flops_matched"] = dense_point(w, d, dev, sh, ev)
            res["dense_flops_matched"]["grouped_step_us"] = round(ph["step_events_us"], 2)

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(w, d, args.cpu_seconds)
        log("[bench] timing the CPU oracle on one thread")
        res["cpu_baseline"]["single_thread"] = cpu_single_thread()
    ev.close()
    line = json.dumps(res)
    print(line, flush=True)
    if args.report:
        with open(args.report, "w") as fh:
            fh.write(line + "\n")


if __name__ == "__main__":
    main()
