#!/usr/bin/env python3
"""Benchmark of the PowerSGD step (compress + finite check + decompress/error update) on one
MI355X, on the 64-resblock d_model=3968 per-GPU gradient shard at rank 112.

    python bench.py [--steps K] [--warmup W] [--workload 3] [--no-out] [--no-cpu-baseline]

Prints ONE JSON line. `value` is gradient GB/s: the fp16 gradient bytes of the whole shard
(256 matrices, 1.51e9 elements, 3.02 GB) times K, over the wall time of K steps bracketed by
device synchronisation, inputs resident in HBM. Per-kernel durations come from HIP events the
library records around each launch on the step's stream (psgd_profile_events), over the same
timed steps. The `roofline` object is for the streaming kernel with the longest average
duration. `cpu_baseline` times the float64 oracle on a bounded sample of the same workload
(whole resblocks, on this host's cores). `traffic` (HBM bytes per launch) and `mfma` (per
multiplying kernel: MFMA flops per launch and the fraction of cycles its MFMA units were busy)
come from the rocprofv3 counter runs summarised under profiles/; they are reported only while
the library's HIP sources hash to the value recorded there. `mfma.achieved_tflops` divides
the counted flops by the live kernel duration.

One GPU only: --gpus above 1 exits with an error (the path has no multi-GPU leg here; the factor
all-reduces are the identity on one GPU).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "gradient GB/s compressed+decompressed (rank 112) and % HBM roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# algorithmic bytes per gradient element of each streaming kernel (gradient dtype size g):
#   ef_mq       reads G and E                         g + 4
#   mtp         reads G and E again                   g + 4
#   decompress  reads G and E, writes E (and D)       g + 8 (+ 4), plus the q commit (4 n r
#               bytes per matrix: q <- q_next)
STREAMING = ("ef_mq", "mtp", "decompress")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=(2, 3, 4, 5))
    ap.add_argument("--n-blocks", type=int, default=None, help="resblocks of workload 3 (default 64)")
    ap.add_argument("--rank", type=int, default=None, help="override the workload's rank")
    ap.add_argument("--no-out", action="store_true", help="do not write the decompressed gradient")
    ap.add_argument("--inplace", action="store_true",
                    help="in-place form: backprop has accumulated s_b G into the error buffers, so "
                         "no gradient is read (value still counts the fp16 gradient bytes the "
                         "step replaces)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the CPU oracle sample (whole resblocks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 2 GiB (reads 2 GiB, writes 2 GiB) three "
                         "times; under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE scale the "
                         "traffic counters of the library kernels")
    ap.add_argument("--block-scaling", action="store_true",
                    help="only measure the block-boundary gradient scaling calls "
                         "(psgd_block_grad_enter / _exit) on residual-stream gradients of one and "
                         "of 16 sequences (1280 tokens x d_model 3968 each); one JSON line")
    ap.add_argument("--adam", action="store_true",
                    help="only time the step with the optimizer: compress, finite check, global "
                         "norm and clipping, the decompression fused with the Adam update of every "
                         "matrix (16-bit parameters, bf16 and ue8m8 moments) and fp32 Adam on the "
                         "pass-through tensors; one JSON line")
    ap.add_argument("--graph", action="store_true",
                    help="only time the step captured once as a HIP graph and replayed (compress, "
                         "device-side finite check, decompress/update); one JSON line")
    ap.add_argument("--trace-summary", metavar="CSV", default=None,
                    help="only summarise a rocprofv3 --kernel-trace CSV: launches, average and "
                         "per-step time of each library kernel")
    ap.add_argument("--pmc-summary", metavar="DIR", default=None,
                    help="only summarise rocprofv3 --pmc CSV output found under DIR: pmc_FETCH_SIZE/, "
                         "pmc_WRITE_SIZE/ (bench runs) with pmccopy_FETCH_SIZE/, "
                         "pmccopy_WRITE_SIZE/ (copy calibration runs) give per-kernel HBM bytes "
                         "per launch; pmc_MFMA/ MFMA use; pmc_LDS/ LDS bank conflicts")
    return ap.parse_args(argv)


# ------------------------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters
# ------------------------------------------------------------------------------------------
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_64rb_r112.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "pmc_mfma_64rb_r112.txt")
# library kernel (name before any template arguments) -> profiling slot
KERNEL_SLOT = {"k_ef_mq": "ef_mq", "k_mtp": "mtp", "k_decomp": "decompress", "k_gs_gram": "gs_gram",
               "k_gs_factor": "gs_factor", "k_gs_apply_s": "gs_apply", "k_gs_apply": "gs_apply"}
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f64": 78.6}
COPY_BYTES = 1 << 31          # the calibration copy reads and writes 2 GiB per launch


def kernel_source_hash() -> str:
    """sha256 over the code of the library's HIP sources (line comments and blank lines left
    out, so that comment edits keep recorded counters valid): counters taken on other code are
    stale."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "rank_gradient_compression_powersgd_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h")):
            with open(f, encoding="utf-8") as fh:
                code = [ln.split("//", 1)[0].rstrip() for ln in fh]
            h.update(os.path.basename(f).encode() + b"\0" + "\n".join(c for c in code if c).encode())
    return h.hexdigest()[:16]


def _short_kernel(name: str) -> str:
    import re
    name = name.replace("psgd::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


def _pmc_values(path: str, counter: str):
    """{kernel name: {dispatch id: counter value}} of one counter run."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            k = _short_kernel(row["Kernel_Name"])
            vals.setdefault(k, {})[row["Dispatch_Id"]] = float(row["Counter_Value"])
    return vals


def _pmc_means(path: str, counter: str):
    """Mean counter value (KiB, as rocprofv3 reports these counters) per kernel name."""
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in _pmc_values(path, counter).items()}


def pmc_summary(d: str) -> int:
    """Summarise the counter runs found under d: HBM traffic (pmc_FETCH_SIZE/, pmc_WRITE_SIZE/
    with the copy calibration in pmccopy_FETCH_SIZE/, pmccopy_WRITE_SIZE/), MFMA use
    (pmc_MFMA/) and LDS bank conflicts (pmc_LDS/)."""
    done = False
    if os.path.isdir(os.path.join(d, "pmc_FETCH_SIZE")):
        if traffic_summary(d):
            return 1
        done = True
    if os.path.isdir(os.path.join(d, "pmc_MFMA")):
        mfma_summary(os.path.join(d, "pmc_MFMA"))
        done = True
    if os.path.isdir(os.path.join(d, "pmc_LDS")):
        lds_summary(os.path.join(d, "pmc_LDS"))
        done = True
    if not done:
        print(f"no counter runs under {d}", file=sys.stderr)
        return 1
    return 0


def traffic_summary(d: str) -> int:
    fe = _pmc_means(os.path.join(d, "pmc_FETCH_SIZE"), "FETCH_SIZE")
    wr = _pmc_means(os.path.join(d, "pmc_WRITE_SIZE"), "WRITE_SIZE")
    cf = _pmc_means(os.path.join(d, "pmccopy_FETCH_SIZE"), "FETCH_SIZE")
    cw = _pmc_means(os.path.join(d, "pmccopy_WRITE_SIZE"), "WRITE_SIZE")
    # the calibration copy: the elementwise kernel launched three times on 2 GiB
    ck = [k for k in cf if "elementwise" in k and cf[k][1] >= 3]
    if not ck:
        print("no calibration copy kernel found", file=sys.stderr)
        return 1
    f_copy = max(cf[k][0] for k in ck) * 1024.0
    w_copy = max(cw[k][0] for k in cw if "elementwise" in k) * 1024.0
    sf, sw = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    print(f"calibration copy (2 GiB read, 2 GiB written per launch): FETCH_SIZE reads "
          f"{f_copy / 2**30:.3f} GiB -> scale {sf:.3f}; WRITE_SIZE reads {w_copy / 2**30:.3f} GiB -> "
          f"scale {sw:.3f}")
    numel = 1511522304
    # the factors each kernel reads or writes once (fp32, rank 112): sum of m x r and of n x r
    sm, sn = 4 * 112 * 666624, 4 * 81772544
    algo = {"k_ef_mq": 6 * numel + sn + sm, "k_mtp": 6 * numel + sm + sn, "k_decomp": 14 * numel + sm + 2 * sn}
    print(f"{'kernel':34s} {'launches':>8s} {'fetch GB':>9s} {'write GB':>9s} {'total GB':>9s} "
          f"{'algorithmic GB':>15s} {'ratio':>6s}")
    for k in sorted(fe):
        if not k.startswith("k_"):
            continue
        f = fe[k][0] * 1024.0 * sf
        w = wr.get(k, (0.0, 0))[0] * 1024.0 * sw
        base = k.split("<")[0]
        a = algo.get(base)
        print(f"{k:34s} {fe[k][1]:8d} {f / 1e9:9.3f} {w / 1e9:9.3f} {(f + w) / 1e9:9.3f} "
              f"{(a / 1e9 if a else float('nan')):15.3f} {((f + w) / a if a else float('nan')):6.3f}")
        if base in ("k_ef_mq", "k_mtp", "k_decomp"):
            print(f"TRAFFIC {KERNEL_SLOT[base]} {int(f + w)} fetch {int(f)} write {int(w)} source {kernel_source_hash()}")
    return 0


def mfma_summary(mf: str) -> None:
    busy = _pmc_values(mf, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _pmc_values(mf, "GRBM_GUI_ACTIVE")
    mops = {t: _pmc_values(mf, f"SQ_INSTS_VALU_MFMA_MOPS_{t.upper()}") for t in ("bf16", "f16", "f64")}
    print()
    print("MFMA counters, mean over the launches that multiply (a second-pass launch that returns at")
    print("once is left out): busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs);")
    print("flops = 512 x SQ_INSTS_VALU_MFMA_MOPS_<type>")
    print(f"{'kernel':34s} {'launches':>8s} {'busy':>6s} {'bf16 GFLOP':>11s} {'f16 GFLOP':>10s} {'f64 GFLOP':>10s}")
    for k in sorted(busy):
        if not k.startswith("k_") or k not in gui:
            continue
        ids = [i for i in busy[k] if sum(mops[t].get(k, {}).get(i, 0.0) for t in mops) > 0]
        if not ids:
            continue
        cyc = sum(gui[k][i] for i in ids) / 8.0
        frac = sum(busy[k][i] for i in ids) / (cyc * 1024.0) if cyc > 0 else 0.0
        fl = {t: sum(mops[t].get(k, {}).get(i, 0.0) for i in ids) / len(ids) * 512.0 for t in mops}
        print(f"{k:34s} {len(ids):8d} {frac:6.3f} {fl['bf16'] / 1e9:11.1f} {fl['f16'] / 1e9:10.1f} "
              f"{fl['f64'] / 1e9:10.1f}")
        base = k.split("<")[0]
        if base in KERNEL_SLOT and any(fl.values()):
            print(f"MFMA {KERNEL_SLOT[base]} busy {frac:.4f} bf16 {int(fl['bf16'])} f16 {int(fl['f16'])} "
                  f"f64 {int(fl['f64'])} source {kernel_source_hash()}")


def lds_summary(ld: str) -> None:
    conf = _pmc_values(ld, "SQ_LDS_BANK_CONFLICT")
    act = _pmc_values(ld, "SQ_LDS_IDX_ACTIVE")
    insts = _pmc_values(ld, "SQ_INSTS_LDS")
    print()
    print("LDS counters, summed over the launches that use LDS: conflict = SQ_LDS_BANK_CONFLICT /")
    print("SQ_LDS_IDX_ACTIVE (share of the cycles the LDS spent on indexed accesses that were bank-")
    print("conflict stalls); instructions = SQ_INSTS_LDS per launch")
    print(f"{'kernel':34s} {'launches':>8s} {'conflict':>9s} {'active Mcyc':>12s} {'LDS Minst':>10s}")
    for k in sorted(act):
        if not k.startswith("k_"):
            continue
        ids = [i for i in act[k] if act[k][i] > 0]
        if not ids:
            continue
        a = sum(act[k][i] for i in ids)
        c = sum(conf.get(k, {}).get(i, 0.0) for i in ids)
        n = sum(insts.get(k, {}).get(i, 0.0) for i in ids) / len(ids)
        print(f"{k:34s} {len(ids):8d} {c / a:9.3f} {a / len(ids) / 1e6:12.2f} {n / 1e6:10.2f}")


def trace_summary(path: str) -> int:
    """Per-kernel table of a rocprofv3 --kernel-trace CSV (library kernels only). Steps are
    counted by the finite check, which runs once per step; k_gemm_nt, launched twice per step
    (M q, then M^T P_hat), is split by launch order."""
    import csv
    rows = []
    for row in csv.DictReader(open(path)):
        if "psgd::" not in row["Kernel_Name"]:
            continue
        rows.append((int(row["Start_Timestamp"]), _short_kernel(row["Kernel_Name"]),
                     (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3))
    rows.sort()
    steps = sum(1 for r in rows if r[1] == "k_check_finite")
    if steps == 0:
        print("no library step in the trace", file=sys.stderr)
        return 1
    per = {}
    gemm = 0
    for _, k, us in rows:
        if k == "k_gemm_nt":
            k = "k_gemm_nt (M q)" if gemm % 2 == 0 else "k_gemm_nt (M^T P_hat)"
            gemm += 1
        per.setdefault(k, []).append(us)
    tot = sum(sum(v) for v in per.values())
    print(f"{steps} steps (warm-up included), {len(rows)} library kernel launches")
    print("| kernel | launches | average us | ms per step | share |")
    print("|---|---|---|---|---|")
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {k} | {len(v)} | {sum(v) / len(v):.1f} | {sum(v) / steps / 1e3:.3f} | "
              f"{100 * sum(v) / tot:.1f}% |")
    print(f"| all library kernels | {len(rows)} | | {tot / steps / 1e3:.3f} | |")
    return 0


def factor_bytes(kernel: str, w) -> int:
    """Bytes of the low-rank factors a streaming kernel must read or write once per launch (fp32,
    r = the workload's rank): M Q reads q (n x r) and writes P (m x r); M^T P reads P^T (m x r,
    as two 16-bit halves) and writes q_next (n x r); the decompression reads P (m x r) and q_next
    (n x r) and writes q <- q_next (n x r)."""
    sm = sum(spec.m for spec in w.matrices) * w.rank * 4
    sn = sum(spec.n for spec in w.matrices) * w.rank * 4
    return {"ef_mq": sn + sm, "mtp": sm + sn, "decompress": sm + 2 * sn}[kernel]


def recorded_mfma(slot: str):
    """{"busy": fraction, dtype: flops per launch} of a kernel from the MFMA counter run, or None
    when absent or taken on other kernel sources."""
    try:
        lines = open(MFMA_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) == 12 and f[0] == "MFMA" and f[1] == slot and f[11] == kernel_source_hash():
            return {"busy": float(f[3]), "bf16": int(f[5]), "f16": int(f[7]), "f64": int(f[9])}
    return None


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` recorded from the counter runs, or None when absent or
    taken on other kernel sources."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) >= 9 and f[0] == "TRAFFIC" and f[1] == kernel and f[8] == kernel_source_hash():
            return int(f[2])
    return None


class Hip:
    """The few HIP runtime calls the timing needs (the runtime torch already loaded)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        h = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(h)) == 0
        return h.value

    def record(self, ev: int, stream: int):
        assert self.lib.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a: int, b: int):
        """Milliseconds between two recorded events; None when either was never recorded (a
        profiling slot whose kernel the step did not launch)."""
        ms = ctypes.c_float()
        err = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        return float(ms.value) if err == 0 else None

    def destroy(self, ev: int):
        self.lib.hipEventDestroy(ev)


def workload_name(config: int, w, numel: int) -> str:
    shapes = []
    for s in w.matrices:
        kind = s.name.split(".")[-1]
        if all(k != kind for k, _ in shapes):
            shapes.append((kind, f"{s.m}x{s.n}"))
    what = ", ".join(f"{k} {mn}" for k, mn in shapes)
    share = ("unsharded d_model=3968 resblock" if config == 5
             else f"{w.n_blocks}-resblock d_model=3968 per-GPU shard")
    return (f"{share}: {len(w.matrices)} {w.dtype} matrices ({what}), {numel} elements, "
            f"rank {w.rank}")


def build_workload(config: int, n_blocks, write_out: bool, inplace: bool = False, rank=None):
    import dataclasses
    import torch
    import workloads as wl
    from rank_gradient_compression_powersgd_amd import PowerSGDGroup
    w = wl.workload(config, n_blocks) if config == 3 else wl.workload(config)
    if rank is not None:
        w = dataclasses.replace(w, rank=rank)
    dev = torch.device("cuda", 0)
    grads, q0 = [], []
    for s in w.matrices:
        grads.append(wl.gradient_torch(w, s, 0, dev))
        q0.append(wl.initial_q_torch(w, s, dev, w.rank))
    scale = torch.tensor(wl.scales_np(w), device=dev)
    err = None
    if inplace:
        # the error buffers hold M = s_b G (zero previous error); no gradient tensors remain
        err = [g.float().mul_(float(scale[s.block])) for g, s in zip(grads, w.matrices)]
        grads = [None] * len(grads)
        torch.cuda.empty_cache()
    group = PowerSGDGroup(grads, [s.block for s in w.matrices], scale, w.rank, q0, err, write_out)
    passthrough = [torch.from_numpy(wl.passthrough_np(config, w.n_blocks)).to(dev).reshape(-1)]
    torch.cuda.synchronize()
    return w, group, passthrough


def cpu_baseline(seconds: float):
    """The float64 oracle, as it is, on whole resblocks of the same per-GPU shard shapes
    (numpy-generated, rank 112, cold start) until `seconds` of oracle time have passed."""
    import numpy as np
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:  # pragma: no cover
        blas_threads = 0
    w = wl.workload(3)
    per_block = [s for s in w.matrices if s.block == 0]
    t_total, nbytes, blocks = 0.0, 0, 0
    while t_total < seconds and blocks < w.n_blocks:
        specs = [s for s in w.matrices if s.block == blocks]
        grads = [wl.gradient_np(w, s, 0).astype(np.float32) for s in specs]
        errs = [np.zeros((s.m, s.n), np.float32) for s in specs]
        qs = [wl.initial_q_np(w, s) for s in specs]
        t0 = time.perf_counter()
        oracle.step_group(grads, errs, qs, [0] * len(specs), wl.scales_np(w)[blocks:blocks + 1])
        t_total += time.perf_counter() - t0
        nbytes += sum(s.m * s.n * 2 for s in specs)
        blocks += 1
    cores = len(os.sched_getaffinity(0))
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": cores,
            "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"{blocks} of 64 resblocks ({blocks * len(per_block)} matrices, "
                      f"{nbytes / 1e9:.3f} GB fp16 gradient), float64 numpy oracle, cold start, "
                      f"{t_total:.1f} s"}

ADAM_HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
ADAM_MAX_NORM = 1.0


def adam_cpu_baseline(seconds: float, rank: int):
    """The float64 oracles as they are (PowerSGD step, then the optimizer step with 16-bit
    storage) on whole resblocks of the per-GPU shard, cold start, for about `seconds`."""
    import numpy as np
    import oracle
    import workloads as wl
    w = wl.workload(3)
    hp = oracle.AdamHyper(**ADAM_HP)
    t_total, nbytes, blocks = 0.0, 0, 0
    while t_total < seconds and blocks < w.n_blocks:
        specs = [s for s in w.matrices if s.block == blocks]
        grads = [wl.gradient_np(w, s, 0).astype(np.float32) for s in specs]
        errs = [np.zeros((s.m, s.n), np.float32) for s in specs]
        qs = [wl.initial_q_np(w, s, rank) for s in specs]
        states = [oracle.AdamState(np.zeros((s.m, s.n)), np.zeros((s.m, s.n)), np.zeros((s.m, s.n)))
                  for s in specs]
        t0 = time.perf_counter()
        st = oracle.step_group(grads, errs, qs, [0] * len(specs), wl.scales_np(w)[blocks:blocks + 1])
        oracle.adam_group_step(states, st.D, 0, False, hp, max_norm=ADAM_MAX_NORM)
        t_total += time.perf_counter() - t0
        nbytes += sum(s.m * s.n * 2 for s in specs)
        blocks += 1
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{blocks} of 64 resblocks ({4 * blocks} matrices, {nbytes / 1e9:.3f} GB fp16 "
                      f"gradient): float64 PowerSGD step then float64 Adam with 16-bit storage, "
                      f"cold start, {t_total:.1f} s (the clipping norm over the sampled blocks only)"}


def adam_bench(a, hip) -> int:
    """The step with the optimizer. Per gradient element the fused decompression reads G, E,
    theta, m1, m2 and writes E, theta, m1, m2 (no D): g + 8 + 3 * 2 * p bytes with 2-byte
    moments and p-byte parameters (22 bytes for fp16 gradients and parameters), plus the factors
    it reads (P, q_next) and the q commit."""
    import torch
    import rank_gradient_compression_powersgd_amd as psgd
    w, group, passthrough = build_workload(a.workload, a.n_blocks, False, a.inplace, a.rank)
    dev = torch.device("cuda", 0)
    pdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    params, m1s, m2s = [], [], []
    for i, s in enumerate(w.matrices):
        g = torch.Generator(device=dev)
        g.manual_seed(11_000 + i)
        params.append((torch.randn((s.m, s.n), generator=g, device=dev) * 0.02).to(pdt))
        m1s.append(torch.zeros((s.m, s.n), dtype=torch.int16, device=dev))
        m2s.append(torch.zeros((s.m, s.n), dtype=torch.int16, device=dev))
    group.attach_adam(params, m1s, m2s)
    pg = passthrough[0]
    pstate = [(torch.randn_like(pg) * 0.02, torch.zeros_like(pg), torch.zeros_like(pg), pg)]
    hp = psgd.binding.psgd_adam_hparams(**ADAM_HP)
    stream = int(torch.cuda.current_stream().cuda_stream)
    nslot = len(psgd.PROFILE_SLOTS)
    for _ in range(a.warmup):
        group.step_adam(hp, pstate, None, ADAM_MAX_NORM)
    torch.cuda.synchronize()
    K = a.steps
    kev = [[hip.event() for _ in range(2 * nslot)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        psgd.psgd_profile_events(group.ctx, kev[k])
        group.step_adam(hp, pstate, None, ADAM_MAX_NORM)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    psgd.psgd_profile_events(group.ctx, None)
    assert int(group.skip.item()) == 0, "a timed step was skipped"
    steps_done = int(group.adam_step.item())
    assert steps_done == a.warmup + K, steps_done
    kern = {}
    for j, name in enumerate(psgd.PROFILE_SLOTS):
        vals = [hip.elapsed_ms(kev[k][2 * j], kev[k][2 * j + 1]) for k in range(K)]
        if all(v is not None for v in vals):
            kern[name] = statistics.mean(vals)
    for evs in kev:
        for e in evs:
            hip.destroy(e)
    numel = w.numel
    gsz = 0 if a.inplace else (2 if w.dtype in ("f16", "bf16") else 4)
    psz = params[0].element_size()
    per_elem = gsz + 8 + 2 * (psz + 2 + 2)
    ebytes = per_elem * numel
    nbytes = ebytes + factor_bytes("decompress", w)   # + P and q_next read, q <- q_next written
    gbs = nbytes / (kern["decompress_adam"] * 1e-3) / 1e9
    ms = wall * 1e3 / K
    norm = group.adam_norm.cpu().tolist()
    line = {
        "metric": f"gradient GB/s compressed+decompressed+Adam (rank {w.rank}), 1 MI355X",
        "value": round(w.grad_bytes * K / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": workload_name(a.workload, w, numel), "grad_dtype": w.dtype,
                   "param_dtype": str(pdt).replace("torch.", ""), "moments": "m1 bf16, m2 ue8m8",
                   "passthrough": "gains/biases fp32 Adam", "hparams": ADAM_HP, "max_norm": ADAM_MAX_NORM,
                   "last_norm": round(norm[0], 4), "last_clip": norm[1]},
        "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": nbytes,
                     "bytes_per_element": per_elem, "element_bytes": ebytes, "factor_bytes": nbytes - ebytes,
                     "frac_elements_only": round(ebytes / (kern["decompress_adam"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "avg_ms": round(kern["decompress_adam"], 4), "kernel": "decompress_adam"},
        "cpu_baseline": None,
    }
    group.close()
    del group, params, m1s, m2s
    torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        log("timing the CPU oracles ...")
        line["cpu_baseline"] = adam_cpu_baseline(a.cpu_seconds, w.rank)
    print(json.dumps(line), flush=True)
    return 0


def graph_bench(a) -> int:
    """The step captured once in a HIP graph (no host synchronisation inside) and replayed: the
    same kernels as the eager step without the per-launch host overhead between them."""
    import torch
    w, group, passthrough = build_workload(a.workload, a.n_blocks, not a.no_out, a.inplace, a.rank)
    for _ in range(a.warmup):
        group.step(passthrough)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        group.compress()
        group.check_finite(passthrough)
        group.decompress_update()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(a.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    assert int(group.skip.item()) == 0, "a replayed step was skipped"
    ms = e0.elapsed_time(e1) / a.steps
    numel = sum(sp.m * sp.n for sp in w.matrices)
    print(json.dumps({"metric": "gradient GB/s, step replayed from a HIP graph, 1 MI355X",
                      "value": round(w.grad_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                      "ms_per_step": round(ms, 4), "steps": a.steps, "warmup": a.warmup,
                      "config": {"workload": workload_name(a.workload, w, numel)}}), flush=True)
    group.close()
    return 0


def block_scaling_bench(a) -> int:
    """Per-launch time of the block-boundary scaling calls, HIP events on the launch stream.
    Algorithmic bytes per element: entry reads 4 (fp32) and writes 2 (fp16); exit reads 2 + 4
    and writes 4; the fused boundary (exit of block b, entry of block b - 1) reads 4 + 2 and
    writes 4 + 2. The per-backward figures are 64 resblocks x (entry + exit) at one sequence,
    and the same with the 63 inner boundaries fused."""
    import numpy as np
    import torch
    import rank_gradient_compression_powersgd_amd as psgd
    dev = torch.device("cuda", 0)
    ctx = psgd.psgd_create(0, 1)
    d_model, tokens = 3968, 1280
    scale = torch.tensor([np.float32(2.0 ** 12)], device=dev)
    flag = torch.zeros(1, dtype=torch.uint8, device=dev)
    res = {}
    for seqs in (1, 16):
        n = seqs * tokens * d_model
        g = torch.Generator(device=dev)
        g.manual_seed(7000 + seqs)
        dx = torch.randn(n, generator=g, device=dev).mul_(1e-6)
        out = torch.empty(n, dtype=torch.float16, device=dev)
        acc = torch.zeros(n, dtype=torch.float32, device=dev)
        out2 = torch.empty(n, dtype=torch.float16, device=dev)
        for name, call, bpe in (("enter", lambda: psgd.psgd_block_grad_enter(ctx, dx, scale, out), 6),
                                ("exit", lambda: psgd.psgd_block_grad_exit(ctx, acc, out, scale, flag), 10),
                                ("exit_enter", lambda: psgd.psgd_block_grad_exit_enter(ctx, acc, out, scale, scale, out2, flag), 12)):
            for _ in range(a.warmup):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(a.steps):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / a.steps
            gbs = bpe * n / (us * 1e-6) / 1e9
            res[f"{name}_{seqs}seq"] = {"elements": n, "us": round(us, 2), "GB/s": round(gbs, 1),
                                        "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_element": bpe}
    psgd.psgd_destroy(ctx)
    # the oracle on one sequence (entry + exit), on this host's cores
    import oracle
    rng = np.random.default_rng(7001)
    x = (rng.standard_normal(tokens * d_model) * 1e-6).astype(np.float32)
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 5.0:
        h = oracle.block_grad_enter(x, 4096.0, "f16")
        oracle.block_grad_exit(np.zeros_like(x), h, 4096.0, "f16")
        reps += 1
    cpu_s = (time.perf_counter() - t0) / reps
    big = res["exit_16seq"]
    line = {
        "metric": "block-boundary gradient scaling GB/s (algorithmic bytes), 1 MI355X",
        "value": big["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "higher_is_better": True, "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "residual-stream gradient at resblock boundaries: 1280 tokens x "
                               "d_model 3968 per sequence, 1 and 16 sequences, S_b = 2^12"},
        "ops": res,
        "backward_pass_us_1seq": round(64 * (res["enter_1seq"]["us"] + res["exit_1seq"]["us"]), 1),
        "backward_pass_us_1seq_fused": round(res["enter_1seq"]["us"] + 63 * res["exit_enter_1seq"]["us"]
                                             + res["exit_1seq"]["us"], 1),
        "roofline": {"bound": "hbm", "achieved": big["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": big["frac"], "traffic": None, "kernel": "k_block_exit, 16 sequences"},
        "cpu_baseline": {"value": round(10 * tokens * d_model / cpu_s / 1e9, 3), "unit": "GB/s",
                         "cores": 1, "kind": "oracle",
                         "sample": f"entry + exit of one sequence ({tokens * d_model} elements), "
                                   f"numpy float64, {reps} repetitions in {reps * cpu_s:.1f} s; "
                                   "GB/s of the exit's 10 bytes per element"},
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None) -> int:
    a = parse(argv)
    if a.pmc_summary:
        return pmc_summary(a.pmc_summary)
    if a.trace_summary:
        return trace_summary(a.trace_summary)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {a.gpus}, WORLD_SIZE {world}): the "
              "PowerSGD path here has no multi-GPU leg; run with --gpus 1", file=sys.stderr)
        return 2
    import torch
    import rank_gradient_compression_powersgd_amd as psgd
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if a.copy_calibration:
        x = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"kernel": "elementwise neg", "bytes_read": x.numel() * 4,
                                               "bytes_written": y.numel() * 4, "launches": 3}}))
        return 0
    psgd.load_library()
    if a.block_scaling:
        return block_scaling_bench(a)
    if a.graph:
        return graph_bench(a)
    hip = Hip()
    if a.adam:
        return adam_bench(a, hip)
    log(f"building workload {a.workload} ...")
    w, group, passthrough = build_workload(a.workload, a.n_blocks, not a.no_out, a.inplace, a.rank)
    stream = int(torch.cuda.current_stream().cuda_stream)
    nslot = len(psgd.PROFILE_SLOTS)

    for _ in range(a.warmup):
        group.step(passthrough)
    torch.cuda.synchronize()

    K = a.steps
    kev = [[hip.event() for _ in range(2 * nslot)] for _ in range(K)]
    sev = [(hip.event(), hip.event()) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        psgd.psgd_profile_events(group.ctx, kev[k])
        hip.record(sev[k][0], stream)
        group.step(passthrough)
        hip.record(sev[k][1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    psgd.psgd_profile_events(group.ctx, None)
    assert int(group.skip.item()) == 0, "a timed step was skipped"

    step_ms = sorted(hip.elapsed_ms(s0, s1) for s0, s1 in sev)
    kern = {}
    for j, name in enumerate(psgd.PROFILE_SLOTS):
        vals = [hip.elapsed_ms(kev[k][2 * j], kev[k][2 * j + 1]) for k in range(K)]
        if all(v is not None for v in vals):
            kern[name] = statistics.mean(vals)
    for evs in kev:
        for e in evs:
            hip.destroy(e)
    for s0, s1 in sev:
        hip.destroy(s0)
        hip.destroy(s1)

    gsz = 2 if w.dtype in ("f16", "bf16") else 4
    if a.inplace:
        gsz = 0                        # no gradient is read
    numel = w.numel
    per_elem = {"ef_mq": gsz + 4, "mtp": gsz + 4, "decompress": gsz + 8 + (0 if a.no_out else 4)}
    rooflines = {}
    for name in STREAMING:
        ebytes = per_elem[name] * numel
        fbytes = factor_bytes(name, w)
        nbytes = ebytes + fbytes
        gbs = nbytes / (kern[name] * 1e-3) / 1e9
        rooflines[name] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                           "bytes_per_launch": nbytes, "element_bytes": ebytes, "factor_bytes": fbytes,
                           "frac_elements_only": round(ebytes / (kern[name] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "avg_ms": round(kern[name], 4)}
    if w.rank > 128:
        # Above rank 128 the products are GEMMs on split operands: bound by MFMA, not HBM. The
        # achieved rate counts the method's own flops, 2 m n r per product (the split runs three
        # MFMA products for each), against the dense 16-bit MFMA peak.
        alg = 2 * w.rank * numel
        for name in STREAMING:
            tf = alg / (kern[name] * 1e-3) / 1e12
            rooflines[name] = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS["bf16"],
                               "unit": "TFLOP/s", "frac": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4),
                               "traffic": None, "flops_per_launch": alg, "avg_ms": round(kern[name], 4),
                               "hbm_bytes_per_launch": rooflines[name]["bytes_per_launch"]}
    dom = max(STREAMING, key=lambda n: kern[n])
    counted = (a.workload == 3 and not a.no_out and not a.inplace and a.n_blocks in (None, 64)
               and a.rank in (None, 112))
    mfma = {}
    if counted:
        for name in STREAMING:
            rooflines[name]["traffic"] = recorded_traffic(name)
        # MFMA use of the kernels that multiply, from the counter run on the same sources
        for name in ("ef_mq", "gs_gram", "gs_apply", "mtp", "decompress"):
            rec = recorded_mfma(name)
            if rec is None or name not in kern:
                continue
            dt = max(("bf16", "f16", "f64"), key=lambda t: rec[t])
            tf = rec[dt] / (kern[name] * 1e-3) / 1e12
            mfma[name] = {"dtype": dt, "flops_per_launch": rec[dt], "achieved_tflops": round(tf, 1),
                          "peak_tflops": MFMA_PEAK_TFLOPS[dt], "frac": round(tf / MFMA_PEAK_TFLOPS[dt], 4),
                          "busy": round(rec["busy"], 4)}
    roof = dict(rooflines[dom])
    roof["kernel"] = dom

    ms_per_step = wall * 1e3 / K
    value = w.grad_bytes * K / wall / 1e9
    flops = 6 * w.rank * numel * 3       # three bf16/fp16 products per GEMM, three GEMMs
    line = {
        "metric": METRIC if w.rank == 112 else METRIC.replace("rank 112", f"rank {w.rank}"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": workload_name(a.workload, w, numel),
            "grad_dtype": w.dtype, "rank": w.rank, "matrices": len(w.matrices),
            "mode": "in-place (M accumulated in the error buffer)" if a.inplace else "gradient + error buffer",
            "grad_bytes": w.grad_bytes, "decompressed_out": not a.no_out,
            "arithmetic": "M and E fp32; products as split bf16/fp16 MFMA with fp32 accumulation; "
                          "orthonormalisation fp64",
        },
        "step_ms_median": round(statistics.median(step_ms), 4),
        "step_ms_p90": round(step_ms[min(K - 1, int(math.ceil(0.9 * K)) - 1)], 4),
        "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
        "streaming": rooflines,
        "mfma_equivalent_tflops": round(flops / (ms_per_step * 1e-3) / 1e12, 1),
        "mfma": mfma or None,
        "roofline": roof,
        "cpu_baseline": None,
    }
    group.close()
    del group
    torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(a.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
