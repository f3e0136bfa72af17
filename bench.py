"""Benchmark: block-sparse attention throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one fused block-sparse attention call (SDD -> block-sparse
softmax -> DSD in the fused kernel) over the whole workload, inputs already
resident in HBM and the layout tables built once beforehand. The default
workload is the largest, random_b128_bf16 (Z=1, H=32, N=16384, d=128,
128-blocks, per-head random layouts of density 0.25, bf16 operands). The value is
TFLOP/s over the stored blocks only (4 b^2 d flops per stored block per batch
element). Rank 0 prints one JSON line with, besides the contract fields:
  roofline      the fused kernel's achieved TFLOP/s against the MFMA peak of
                its dtype, timed with HIP events on the stream it runs on;
                `traffic` is the HBM bytes per launch from rocprofv3 counters
                (profiles/traffic_<workload>.txt), null if that file is
                missing or the kernel source changed since it was taken
  cpu_baseline  the oracle (float64 numpy, per-block route) timed on this
                host's cores on a bounded sample of block rows
  ops           the unfused three-call path (SDD, softmax, DSD), the
                standalone DDS where the workload has one, and the one-time
                layout build, each timed on its own after two untimed calls
  kv_share      on a layout with a K/V sharing plan (slope-1 ACSR): the
                plan and the kernel time with and without it, timed in
                alternating rounds (the headline uses the library's default)
  fused_other_workloads
                the fused kernel's time, TFLOP/s and roofline fraction on
                each of the other workloads
Other modes:
  --calibrate-copy   a plain 1 GiB device copy (for scaling HBM counters)
  --all              also print one line per workload to stderr
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

METRIC = "block-sparse attention TFLOP/s on nnz blocks + % of MFMA peak, 1 MI355X"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "fp8": 5033.2}   # MI355X dense MFMA (fp8: twice bf16)
# fused attention with fp8 score operands: half the flops (Q K^T) at the fp8
# peak, half (P V) at the bf16 peak
PEAK_FP8_QK = 1.0 / (0.5 / PEAK_TFLOPS["fp8"] + 0.5 / PEAK_TFLOPS["bf16"])
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "random_b128_bf16"


def _events_time(fn, n, stream):
    """Run fn n times on `stream`; mean ms per call from HIP events recorded
    on that stream."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n


def _source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the sources each dtype's fused kernel is built from (dispatch included): a
# committed traffic figure counts only while they are unchanged
_C = "block_sparse_matmul_amd/csrc/"
ATTN_SOURCES = {
    "f32": [_C + "attention.hip", _C + "rowblock.h", _C + "tile.h", _C + "internal.h"],
    "bf16": [_C + "attention.hip", _C + "attention_wide.hip", _C + "tile.h", _C + "internal.h"],
}


def _traffic(workload, dtype):
    """HBM bytes per launch of the fused kernel from committed counters."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != _source_hash(ATTN_SOURCES[dtype]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_flops(nnz, Z, block, d):
    """FLOPs on stored blocks: 2 b^2 d for the score product plus 2 b^2 d for
    P.V, per stored block and batch entry (masked halves of diagonal blocks
    count)."""
    return 4 * block * block * d * nnz * Z


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(w, lay, q, k, v, budget_s=12.0, seed=0):
    """The oracle's per-block route on a seeded random sample of block rows,
    for about budget_s seconds of wall time; TFLOP/s over the sampled rows'
    stored blocks. `cores` is the number of threads the sample kept busy on
    average (process CPU time over wall time, rounded up), next to the
    host's cores, its CPU model and the size of numpy's BLAS thread pool."""
    import math
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                           or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    rng = np.random.default_rng(seed)
    rows = [(z, h, r) for z in range(w.Z) for h in range(w.H) for r in range(w.nb)]
    order = rng.permutation(len(rows))
    lens = lay.sum(axis=2)
    # the oracle converts its inputs to float64 once per call; hand it the
    # per-head slices it needs so the sample measures the arithmetic
    # block rows in a seeded order until the budget is spent; a workload
    # that finishes sooner is run again from the start
    done_blocks, n_rows = 0, 0
    c0 = time.process_time()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 <= budget_s:
        for i in order:
            z, h, r = rows[i]
            oracle.attention_blockrow(q[z:z + 1, h:h + 1], k[z:z + 1, h:h + 1], v[z:z + 1, h:h + 1],
                                      lay[h:h + 1], w.block, w.scale, w.causal, 0, 0, r)
            done_blocks += int(lens[h, r])
            n_rows += 1
            if time.perf_counter() - t0 > budget_s:
                break
    el = time.perf_counter() - t0
    busy = (time.process_time() - c0) / el
    flops = 4 * w.block * w.block * w.d * done_blocks
    if n_rows <= len(rows):
        what = f"{n_rows} of {len(rows)} block rows of {w.name}"
    else:
        what = f"{n_rows} block-row evaluations, {n_rows / len(rows):.1f} passes over the {len(rows)} block rows of {w.name}"
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": max(1, math.ceil(busy - 0.05)),
            "kind": "oracle",
            "sample": f"{what} ({done_blocks} stored blocks), oracle per-block route in float64 numpy, {el:.1f} s",
            "threads_busy": round(busy, 2), "host_cores": len(os.sched_getaffinity(0)),
            "cpu_count": os.cpu_count(), "cpu_model": _cpu_model(), "blas_threads": blas_threads}


def run_workload(w, steps, warmup, with_ops=True, with_cpu=True):
    import numpy as np
    import torch

    import block_sparse_matmul_amd as bsa
    import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    lay = W.make_layout(w)
    qh, kh, vh = W.make_qkv(w)
    q, k, v = qh.to(dev), kh.to(dev), vh.to(dev)

    def build_layout():
        if w.pattern == "strided_acsr":
            return bsa.Layout.acsr(W.make_acsr(w), w.H, w.nb, w.nb, w.block)
        return bsa.Layout(torch.from_numpy(lay), w.block)

    # The first build pays the library's one-time set-up (module load, first
    # allocations); the second is what every later layout costs.
    t0 = time.perf_counter()
    L = build_layout()
    lut_first_ms = (time.perf_counter() - t0) * 1e3
    del L
    t0 = time.perf_counter()
    L = build_layout()
    lut_ms = (time.perf_counter() - t0) * 1e3
    out = torch.empty_like(q)
    flops = attention_flops(L.nnz, w.Z, w.block, w.d)

    def step():
        bsa.attention(L, q, k, v, w.scale, w.causal, out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kern_ms = _events_time(step, steps, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    tflops = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = _traffic(w.name, w.dtype)
    share = None
    rows, stride = L.kv_share()
    if rows > 1:
        # the fused kernel with and without the K/V sharing across block rows,
        # timed in alternating rounds of 10 calls (a run timed after another
        # starts at a different clock), medians
        t_one, t_sh = [], []
        for r in range(7):
            for on, dst in ((False, t_one), (True, t_sh)):
                L.set_kv_share(on)
                step()
                dst.append(_events_time(step, 10, stream))
        L.set_kv_share(None)
        t_one, t_sh = sorted(t_one)[3], sorted(t_sh)[3]
        share = {"rows": rows, "stride": stride, "one_row_kernel_ms": round(t_one, 4),
                 "shared_kernel_ms": round(t_sh, 4), "speedup": round(t_one / t_sh, 4),
                 "timing": "medians of 7 alternating rounds of 10 calls each"}
    res = {
        "wall_ms": wall_ms, "kernel_ms": kern_ms, "tflops": tflops, "nnz": L.nnz,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "lut_build_ms": round(lut_ms, 3), "lut_build_first_ms": round(lut_first_ms, 3),
    }
    if share:
        res["kv_share"] = share
    if with_ops:
        ops = {}
        if True:
            S = torch.empty((w.Z, L.nnz, w.block, w.block), dtype=torch.float32, device=dev)
            O2 = torch.empty_like(q)
            n = max(3, steps // 2)
            # every op is called twice before its timed window (code object
            # load, first-touch of the buffers), then timed on its own
            for _ in range(2):
                bsa.sdd(L, q, k, out=S)
            t_sdd = _events_time(lambda: bsa.sdd(L, q, k, out=S), n, stream)
            for _ in range(2):
                bsa.softmax(L, S, w.scale, w.causal, out=S)
            t_sm = _events_time(lambda: bsa.softmax(L, S, w.scale, w.causal, out=S), n, stream)
            for _ in range(2):
                bsa.dsd(L, S, v, out=O2)
            t_dsd = _events_time(lambda: bsa.dsd(L, S, v, out=O2), n, stream)
            sbytes = 4 * w.block * w.block * L.nnz * w.Z
            ops["unfused"] = {
                "sdd_ms": round(t_sdd, 4), "softmax_ms": round(t_sm, 4), "dsd_ms": round(t_dsd, 4),
                "total_ms": round(t_sdd + t_sm + t_dsd, 4),
                "tflops": round(flops / ((t_sdd + t_sm + t_dsd) * 1e-3) / 1e12, 3),
                "softmax_gbs": round(2 * sbytes / (t_sm * 1e-3) / 1e9, 1),
                "softmax_hbm_frac": round(2 * sbytes / (t_sm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            }
            del S, O2
            # backward, 10 b^2 d algorithmic flops per stored block (dP, dQ,
            # dK, dV and the recomputed S). Fused: the dQ kernel and the dK dV
            # kernel from the forward's O and row log-sum-exp (S and dP are
            # formed in both, 14 b^2 d executed). Composed: P recomputed by
            # SDD and softmax, dP = SDD(dO, V), softmax gradient, dQ = DSD,
            # dK and dV by DSD^T, with S and P through HBM.
            g = torch.Generator("cpu").manual_seed(1)
            do = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
            fb = 10 * w.block * w.block * w.d * L.nnz * w.Z
            o, lse = bsa.attention(L, q, k, v, w.scale, w.causal, return_lse=True)
            wsd = torch.empty(lse.shape, dtype=torch.float32, device=dev)
            for _ in range(2):
                bsa.attention_backward_fused(L, q, k, v, o, lse, do, w.scale, w.causal, workspace=wsd)
            t_fb = _events_time(lambda: bsa.attention_backward_fused(L, q, k, v, o, lse, do, w.scale, w.causal,
                                                                     workspace=wsd), n, stream)
            ops["backward"] = {"ms": round(t_fb, 4), "tflops": round(fb / (t_fb * 1e-3) / 1e12, 3),
                               "flops": "10 b^2 d per stored block",
                               "kernels": "fused: dQ over block rows; dK and dV over block columns "
                                          "(one kernel for both; with 16-bit operands S is formed once, "
                                          "half its waves each)"}
            del o, lse, wsd
            ws = (torch.empty((w.Z, L.nnz, w.block, w.block), dtype=torch.float32, device=dev),
                  torch.empty((w.Z, L.nnz, w.block, w.block), dtype=torch.float32, device=dev))
            for _ in range(2):
                bsa.attention_backward(L, q, k, v, do, w.scale, w.causal, workspace=ws)
            t_bwd = _events_time(lambda: bsa.attention_backward(L, q, k, v, do, w.scale, w.causal, workspace=ws),
                                 n, stream)
            ops["backward_composed"] = {"ms": round(t_bwd, 4), "tflops": round(fb / (t_bwd * 1e-3) / 1e12, 3)}
            del do, ws
        if w.dtype == "bf16" and w.d == 128:
            # the same workload with Q and K rounded to fp8 (OCP E4M3): the
            # score product on the fp8 matrix cores, P.V in bf16
            f8 = torch.float8_e4m3fn
            q8, k8 = q.float().to(f8), k.float().to(f8)
            o8 = torch.empty_like(v)
            for _ in range(2):
                bsa.attention(L, q8, k8, v, w.scale, w.causal, out=o8)
            t8 = _events_time(lambda: bsa.attention(L, q8, k8, v, w.scale, w.causal, out=o8), max(3, steps // 2),
                              stream)
            ops["fused_fp8_qk"] = {"ms": round(t8, 4), "tflops": round(flops / (t8 * 1e-3) / 1e12, 3),
                                   "peak": round(PEAK_FP8_QK, 1),
                                   "frac": round(flops / (t8 * 1e-3) / 1e12 / PEAK_FP8_QK, 4),
                                   "operands": "Q, K float8_e4m3fn; V, O bf16"}
            del q8, k8, o8
        if w.dds_m:
            A, Sd = W.make_dds_operands(w, L.nnz)
            A, Sd = A.to(dev), Sd.to(dev)
            C = torch.empty((w.Z, w.H, w.dds_m, w.N), dtype=A.dtype, device=dev)
            n = max(3, steps // 2)
            for _ in range(2):
                bsa.dds(L, A, Sd, out=C)
            t_dds = _events_time(lambda: bsa.dds(L, A, Sd, out=C), n, stream)
            fd = 2 * w.block * w.block * w.dds_m * L.nnz * w.Z
            ops["dds"] = {"ms": round(t_dds, 4), "tflops": round(fd / (t_dds * 1e-3) / 1e12, 3),
                          "frac": round(fd / (t_dds * 1e-3) / 1e12 / PEAK_TFLOPS[w.dtype], 4), "M": w.dds_m}
            del A, Sd, C
        res["ops"] = ops
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(w, lay, qh, kh, vh)
    return res


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB, 5 times: the reference point
    for HBM byte counters (expect 1 GiB read + 1 GiB written per copy)."""
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 5}))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true", help="also run every workload (lines on stderr)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline")
    ap.add_argument("--no-ops", action="store_true", help="skip the per-op breakdown")
    ap.add_argument("--no-others", action="store_true", help="skip the fused kernel on the other workloads")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the block-sparse attention kernels on a "
              "single MI355X (sharding across GPUs is not implemented); use --gpus 1",
              file=sys.stderr)
        return 2
    if args.calibrate_copy:
        calibrate_copy()
        return 0

    import torch
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a visible GPU", file=sys.stderr)
        return 1

    w = W.workload(args.workload)
    if args.all:
        for other in W.WORKLOADS:
            r = run_workload(other, max(5, args.steps // 2), args.warmup, with_ops=not args.no_ops, with_cpu=False)
            print(json.dumps({"workload": other.name, **{k: r[k] for k in ("kernel_ms", "tflops", "nnz", "roofline",
                                                                          "ops") if k in r}}),
                  file=sys.stderr, flush=True)
    r = run_workload(w, args.steps, args.warmup, with_ops=not args.no_ops, with_cpu=not args.no_cpu)
    # the fused kernel on every other workload, briefly (roofline fraction
    # of each, so that one line records where every configuration stands)
    others = {}
    if not args.no_others:
        for other in W.WORKLOADS:
            if other.name == w.name:
                continue
            ro = run_workload(other, max(10, args.steps // 2), max(3, args.warmup), with_ops=False, with_cpu=False)
            others[other.name] = {"dtype": other.dtype, "kernel_ms": round(ro["kernel_ms"], 4),
                                  "tflops": ro["roofline"]["achieved"], "frac": ro["roofline"]["frac"],
                                  "traffic": ro["roofline"]["traffic"], "nnz": ro["nnz"]}
            if ro.get("kv_share"):
                others[other.name]["kv_share"] = ro["kv_share"]
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded layouts and N(0,1) Q/K/V, see workloads/)",
        "config": {"workload": w.name, "Z": w.Z, "H": w.H, "N": w.N, "d": w.d, "block": w.block,
                   "causal": w.causal, "nnz": r["nnz"], "density": round(r["nnz"] / (w.H * w.nb * w.nb), 4),
                   "global_batch": w.Z, "seq_len": w.N, "parallelism": "single GPU"},
        "roofline": r["roofline"],
        "mfma_peak_frac": r["roofline"]["frac"],
        "cpu_baseline": r.get("cpu_baseline"),
        "ops": r.get("ops"),
        "kv_share": r.get("kv_share"),
        "fused_other_workloads": others or None,
        "lut_build_ms": r["lut_build_ms"],
        "lut_build_first_ms": r["lut_build_first_ms"],
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
