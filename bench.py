"""Benchmark: fused RHT + E1M2 row+column quantization of an 8192x2048 bf16
activation on one MI355X, reported as HBM GB/s (algorithmic bytes / time).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-warm] [--copy]
                [--schedule auto|two-pass|single-pass] [--no-extra] [--workload NAME]

A step is one ufp4_quantize_rowcol call (every stage of the hot path: load,
random signs, 16-point Walsh-Hadamard transform, tensor and block maxima,
E4M3 block scales, E1M2 round-to-nearest-even, nibble packing, row-wise and
column-wise stores) on one synthetic activation tensor already resident in
HBM.  Steps rotate over enough input/output buffer sets (>= 600 MB) that the
256 MB Infinity Cache cannot hold the next step's input.

Algorithmic bytes per call: 2 B/element read (bf16) + 2 x 0.5 B/element codes
+ 2 x 1/16 B/element E4M3 scales + 2 x 4 B tensor scales.

The default schedule for this call is the single pass: one kernel that
keeps each tile on chip (the column-wise transform in registers, the raw
rows in LDS) while the tile maxima are exchanged device-wide, so the input
is read once.  The two-pass schedule (tensor-maximum kernel, then a
quantization kernel that reads the input again) is timed beside it.  The
roofline object describes the dominant kernel (the single-pass kernel, i.e.
the whole call; or the two-pass quantization kernel under --schedule
two-pass): its algorithmic bytes per launch are the call's (input once, all
outputs), and its duration is the mean of hipEvent intervals recorded on the
launch stream around that kernel alone, over calls that rotate through the
buffer sets.

The oracle leg (cpu_baseline) times the single-threaded CPU oracle on the same
tensor (row-wise and column-wise), a reported baseline only.

Reported beside the headline, under "extra" (never as the value): a
bandwidth reference on the same buffers (ufp4_roof_rowcol: the quantization
kernels' loads and the call's output bytes with no arithmetic), the RHT-off
call, the E2M1, INT4 and MX32 variants of the call, the other schedule,
delayed scaling, the consumer GEMM (NV16 on the fp16 MFMA; MX32 on the scaled
f8f6f4 MFMA), a streaming
copy of 512 MiB on the same box, the weight workload's shrinkage sweep (SQNR,
mean signed error in grid units and gain alpha per grid, RHT on and off),
the output-gradient workload (stochastic rounding, row+col) and MoE workload
(grouped, row+col; grouped delayed scaling) call times, and the compounding of the GEMM gain through
16 quantized layers.
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

METRIC = "HBM GB/s (% of peak) fused RHT+E1M2 quant, row+col, 8192×2048 bf16"
PEAK_GBPS = 8000.0  # MI355X HBM3E
ROWS, COLS = 8192, 2048
COUNTERS = os.path.join(ROOT, "profiles", "counters_activation_8192x2048.json")
CSRC = os.path.join(ROOT, "fp4_quantization_amd", "csrc")


def algorithmic_bytes(rows: int, cols: int) -> int:
    n = rows * cols
    return 2 * n + 2 * (n // 2) + 2 * (n // 16) + 2 * 4


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic(single: bool):
    """HBM bytes per launch of the dominant kernel and per call under the
    schedule, from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; else (None, None)."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None, None
    if c.get("kernel_source_sha256") != kernel_source_sha():
        return None, None
    h = c.get("hbm_bytes", {})
    if single:
        return h.get("single_pass_kernel"), h.get("single_pass_kernel")
    return h.get("two_pass_quant_kernel"), h.get("two_pass_call")


SINGLE_KERNEL = "ufp4_single_kernel<0, false, true>"
DELAYED_KERNEL = "ufp4_delayed_kernel<0, false, true>"
AMAX_KERNEL = "ufp4_amax_kernel<true>"
QUANT_KERNEL = "ufp4_quant_kernel<0, false, false, true>"
ROOF_KERNEL = "ufp4_roof_kernel"


def _counter_means(csv_dir, counter, counts=None):
    """Mean counter value (KiB) per dispatch, by kernel name, from a rocprofv3
    --pmc CSV directory; also the largest-grid copyBuffer dispatches'.  The
    number of dispatches per kernel goes to `counts` if given."""
    import csv
    import glob

    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {csv_dir}")
    sums, copies = {}, {}
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name, v = r["Kernel_Name"], float(r["Counter_Value"])
                if "copyBuffer" in name:
                    copies.setdefault(int(r["Grid_Size"]), []).append(v)
                else:
                    sums.setdefault(name, []).append(v)
    means = {k: sum(v) / len(v) for k, v in sums.items()}
    if counts is not None:
        counts.update({k: len(v) for k, v in sums.items()})
    copy_mean = None
    if copies:
        big = copies[max(copies)]
        copy_mean = sum(big) / len(big)
    return means, copy_mean


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, commands, workload=None):
    """Write the counter summary bench.py reads: HBM bytes per launch of the
    single-pass kernel, of the two-pass quantization kernel and per two-pass
    call, each counter scaled by what it reads for a plain 512 MiB device
    copy."""
    ncall = {}
    fetch, _ = _counter_means(fetch_dir, "FETCH_SIZE", ncall)
    write, _ = _counter_means(write_dir, "WRITE_SIZE")
    _, copy_fetch = _counter_means(copy_fetch_dir, "FETCH_SIZE")
    _, copy_write = _counter_means(copy_write_dir, "WRITE_SIZE")
    copy_kib = 512 * 1024
    ff, wf = copy_kib / copy_fetch, copy_kib / copy_write
    if workload:
        # the kernels every call launches (at least half as often as the
        # most frequent one); set-up kernels run once or twice per process
        most = max(ncall.values())
        fetch = {k: v for k, v in fetch.items() if 2 * ncall[k] >= most}
        summarize_workload_counters(workload, fetch, write,
                                    {"copy_bytes": copy_kib * 1024, "fetch_kib_raw": copy_fetch,
                                     "write_kib_raw": copy_write, "fetch_factor": ff, "write_factor": wf},
                                    ff, wf, commands)
        return

    def pick(d, key):
        hits = [k for k in d if key in k]
        if len(hits) != 1:
            raise SystemExit(f"kernel {key!r}: found {hits}")
        return hits[0], d[hits[0]]

    kf, ff_ = pick(fetch, SINGLE_KERNEL)
    ka, fa = pick(fetch, AMAX_KERNEL)
    kq, fq = pick(fetch, QUANT_KERNEL)
    _, wf_ = pick(write, SINGLE_KERNEL)
    _, wa = pick(write, AMAX_KERNEL)
    _, wq = pick(write, QUANT_KERNEL)
    kd, fd = pick(fetch, DELAYED_KERNEL)
    _, wd = pick(write, DELAYED_KERNEL)
    kr, fr = pick(fetch, ROOF_KERNEL)
    _, wr = pick(write, ROOF_KERNEL)
    roof = (fr * ff + wr * wf) * 1024
    delayed = (fd * ff + wd * wf) * 1024
    fused = (ff_ * ff + wf_ * wf) * 1024
    quant = (fq * ff + wq * wf) * 1024
    call = quant + (fa * ff + wa * wf) * 1024
    out = {"fetch_kib_raw": {kf: ff_, ka: fa, kq: fq, kd: fd, kr: fr},
           "write_kib_raw": {kf: wf_, ka: wa, kq: wq, kd: wd, kr: wr},
           "copy_calibration": {"copy_bytes": copy_kib * 1024, "fetch_kib_raw": copy_fetch,
                                "write_kib_raw": copy_write, "fetch_factor": ff, "write_factor": wf},
           "hbm_bytes": {"single_pass_kernel": round(fused), "two_pass_quant_kernel": round(quant),
                         "two_pass_call": round(call), "delayed_kernel": round(delayed),
                         "roof_kernel": round(roof)},
           "algorithmic_bytes_per_call": algorithmic_bytes(ROWS, COLS),
           "kernel_source_sha256": kernel_source_sha(), "commands": commands,
           "note": "KiB per dispatch, mean over dispatches; bytes = (fetch * fetch_factor + "
                   "write * write_factor) * 1024; FETCH_SIZE counts traffic beyond L2 (HBM and "
                   "Infinity Cache)"}
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def workload_bytes(name: str) -> int:
    """Algorithmic bytes per call of a named workload (as workload_leg)."""
    if name == "output_grad_16384x4096_sr":
        R, C = 16384, 4096
        return 2 * R * C + R * C + 2 * R * C // 16 + 8
    import synth
    counts = synth.moe_counts(8192, 64, 8, seed=4)
    Rm, Rp, E = int(counts.sum()), int(sum((int(m) + 15) // 16 * 16 for m in counts)), 64
    nbytes = 2 * Rm * 4096 + Rm * 4096 // 2 + Rm * 4096 // 16 + 4096 * Rp // 2 + 4096 * Rp // 16 + 2 * E * 4
    return nbytes + (2 * E * 8 if name.endswith("delayed") else 0)


def summarize_workload_counters(name, fetch, write, copy_cal, ff, wf, commands):
    """Counter summary of a --workload run: calibrated HBM bytes per dispatch
    of every kernel the call launches, and per call."""
    per = {k: round((fetch[k] * ff + write.get(k, 0.0) * wf) * 1024) for k in fetch}
    alg = workload_bytes(name)
    out = {"workload": name, "hbm_bytes_per_dispatch": per, "hbm_bytes_per_call": sum(per.values()),
           "algorithmic_bytes_per_call": alg, "traffic_over_algorithmic": round(sum(per.values()) / alg, 4),
           "fetch_kib_raw": fetch, "write_kib_raw": write, "copy_calibration": copy_cal,
           "kernel_source_sha256": kernel_source_sha(), "commands": commands,
           "note": "KiB per dispatch, mean over dispatches; bytes = (fetch * fetch_factor + write * write_factor) "
                   "* 1024; the kernels each call launches (set-up kernels that run once are left out)"}
    path = os.path.join(ROOT, "profiles", f"counters_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def time_eager(torch, fns, steps, warmup, stream):
    """Back-to-back launches from the host (prebuilt ctypes arguments)."""
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fns[i % len(fns)]()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_graph(torch, fns, steps, warmup, stream):
    """The same K calls captured once in a HIP graph and replayed, so host
    launch overhead cannot starve the GPU."""
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            fns[i % len(fns)]()
    torch.cuda.synchronize()
    g.replay()  # untimed replay
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, g


def cpu_baseline(xb, min_seconds: float = 10.0):
    """The oracle (single-threaded C) on the whole tensor, row-wise then
    column-wise, repeated for at least min_seconds, on one host core."""
    import oracle

    oracle.lib()  # build/load before timing
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        cfg = oracle.config(grid=0, rounding=0, scaling=0, rht=1, rht_seed=1)
        n_calls, t0 = 0, time.perf_counter()
        while True:
            oracle.quantize(xb, cfg, oracle.LAYOUT_ROW)
            oracle.quantize(xb, cfg, oracle.LAYOUT_COL)
            n_calls += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    finally:
        os.sched_setaffinity(0, allowed)
    per_call = dt / n_calls
    return {"value": round(algorithmic_bytes(*xb.shape) / per_call / 1e9, 6), "unit": "GB/s",
            "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
            "elements_per_s": round(xb.size / per_call, 1),
            "sample": f"{n_calls} full row+col oracle calls on the same 8192x2048 tensor, "
                      f"{per_call:.3f} s each, one thread pinned to host core {core} "
                      f"of {os.cpu_count()}"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_bench(torch, args):
    """Plain device-to-device copy of 512 MiB (read 512 MiB + write 512 MiB per
    step): a reference bandwidth, and the known-size kernel that calibrates
    the FETCH_SIZE / WRITE_SIZE counters."""
    n = 512 * 1024 * 1024 // 4
    bufs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(4)]
    for b in bufs:
        b.fill_(1.0)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        bufs[(2 * i + 1) % 4].copy_(bufs[(2 * i) % 4])
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(args.steps):
        bufs[(2 * i + 1) % 4].copy_(bufs[(2 * i) % 4])
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"copy_bytes_per_step": 2 * n * 4, "ms_per_step": round(ms, 6),
                      "copy_gbps": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)


def variant_legs(torch, F, sets, stream, steps):
    """Call times of the comparator variants on the headline tensor and its
    rotating buffer sets: the E2M1 and INT4 grids (NV16) and MX32 scaling
    (one kernel: no tensor maximum), all with the RHT, row+col."""
    import ctypes
    out = {}
    sptr = ctypes.c_void_p(stream.cuda_stream)
    n = ROWS * COLS
    for name, grid, scaling in (("e2m1_nv16", F.GRID_E2M1, F.SCALE_NV16), ("int4_nv16", F.GRID_INT4, F.SCALE_NV16),
                                ("e1m2_mx32", F.GRID_E1M2, F.SCALE_MX32)):
        cfg = F.config(grid, F.ROUND_RTNE, scaling, rht=1, rht_seed=1)
        outs = [(x, F.alloc_layout(ROWS, COLS, scaling, device=x.device), F.alloc_layout(COLS, ROWS, scaling, device=x.device),
                 ws) for x, _, _, ws in sets]
        fns = []
        for x, row, col, ws in outs:
            a = (ctypes.c_void_p(x.data_ptr()), ROWS, COLS, COLS, ctypes.byref(cfg), row.c(), col.c(), ws.ptr, ws.nbytes,
                 sptr)

            def fn(a=a):
                rc = F.lib.ufp4_quantize_rowcol(*a)
                if rc:
                    raise F.Ufp4Error("ufp4_quantize_rowcol", rc)
            fns.append(fn)
        ms, _ = time_graph(torch, fns, steps, 5, stream)
        B = 32 if scaling == F.SCALE_MX32 else 16
        nbytes = 2 * n + n + 2 * (n // B) + 8
        out[f"{name}_rowcol_ms"] = round(ms, 6)
        out[f"{name}_rowcol_gbps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        del outs, fns
    return out


WORKLOADS = ("output_grad_16384x4096_sr", "moe_65536x4096_grouped", "moe_65536x4096_grouped_delayed")


def workload_leg(torch, F, synth, np, dev, stream, name):
    """One call of a named workload other than the headline, on synthetic
    input resident in HBM: (fn, algorithmic bytes per call, elements, the
    buffers to keep alive)."""
    if name == "output_grad_16384x4096_sr":
        # output gradient dY, Laplace + outliers: RHT + E1M2 + stochastic rounding, row+col
        R, C = 16384, 4096
        g = torch.from_numpy(synth.output_grad(R, C, seed=3).view(np.int16)).to(dev)
        c = F.config(F.GRID_E1M2, F.ROUND_STOCHASTIC, F.SCALE_NV16, rht=1, rht_seed=3, sr_seed=3)
        row, col, ws = (F.alloc_layout(R, C, F.SCALE_NV16, device=dev), F.alloc_layout(C, R, F.SCALE_NV16, device=dev),
                        F.Workspace(R, C, device=dev))
        return (lambda: F.ufp4_quantize_rowcol(g, c, row, col, ws, stream),
                2 * R * C + R * C + 2 * R * C // 16 + 8, R * C, (g, row, col, ws, c))
    # MoE activation, 64 ragged expert segments: grouped RHT + E1M2, row+col
    xm, off = synth.moe_activation(8192, 4096, 64, 8, seed=4)
    Rm, E = xm.shape[0], 64
    coff = F.ufp4_grouped_col_offsets(off, 16)
    Rp = int(coff[-1])
    x = torch.from_numpy(xm.view(np.int16)).to(dev)
    offd = torch.from_numpy(off.astype(np.int64)).to(dev)
    c = F.config(F.GRID_E1M2, F.ROUND_RTNE, F.SCALE_NV16, rht=1, rht_seed=4)
    row = F.alloc_layout(Rm, 4096, F.SCALE_NV16, n_tensor_scales=E, device=dev)
    col = F.alloc_layout(4096, Rp, F.SCALE_NV16, n_tensor_scales=E, device=dev)
    ws = F.Workspace(Rm, 4096, E, device=dev)
    nbytes = 2 * Rm * 4096 + Rm * 4096 // 2 + Rm * 4096 // 16 + 4096 * Rp // 2 + 4096 * Rp // 16 + 2 * E * 4
    keep = (x, offd, row, col, ws, c)
    if name == "moe_65536x4096_grouped":
        return lambda: F.ufp4_quantize_grouped(x, offd, Rp, c, row, col, ws, stream), nbytes, Rm * 4096, keep
    if name != "moe_65536x4096_grouped_delayed":
        raise ValueError(name)
    # delayed scaling, chained: each call reads the previous call's
    # per-segment maxima (2 x 4 B per segment in, the same out)
    amax = [torch.full((E, 2), 3.0, dtype=torch.float32, device=dev) for _ in range(2)]
    state = [0]

    def fn():
        i = state[0]
        state[0] ^= 1
        F.ufp4_quantize_grouped_delayed(x, offd, Rp, c, amax[i], amax[i ^ 1], row, col, ws, stream)
    return fn, nbytes + 2 * E * 8, Rm * 4096, keep + (amax,)


def run_workload(torch, F, synth, np, args):
    """Profiler runs of one named workload: warmup + K eager calls, one JSON
    line with the mean call time (so that its kernels' counters and
    durations are not mixed with other tensors')."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)
    fn, nbytes, n_elem, keep = workload_leg(torch, F, synth, np, dev, stream, args.workload)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"workload": args.workload, "steps": args.steps, "ms_per_call": round(ms, 6),
                      "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1), "algorithmic_bytes_per_call": nbytes,
                      "elements": n_elem}), flush=True)


def extra_legs(torch, F, synth, np, dev, stream, steps):
    """Measurements reported beside the headline: a streaming-copy reference
    bandwidth; the weight workload's shrinkage sweep (SQNR, mean signed error
    and gain alpha per grid, RHT on and off); the output-gradient workload
    (SR, row+col) and the MoE workload (grouped, row+col) call times; and the
    compounding of the GEMM gain through a chain of quantized layers; the
    grouped delayed-scaling call on the MoE workload."""
    out = {}
    # streaming copy of 512 MiB on the same box (read + write)
    n = 512 * 1024 * 1024 // 4
    a, b = torch.ones(n, dtype=torch.float32, device=dev), torch.empty(n, dtype=torch.float32, device=dev)
    for _ in range(3):
        b.copy_(a)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(20):
        b.copy_(a)
    s1.record(stream)
    torch.cuda.synchronize()
    out["copy_gbps"] = round(2 * n * 4 / (s0.elapsed_time(s1) / 20 * 1e-3) / 1e9, 1)
    del a, b
    # weight W 2048 x 8192, Student-t(4) tails: the shrinkage sweep per grid
    wb = synth.weight(2048, 8192, seed=2)
    w = torch.from_numpy(wb.view(np.int16)).to(dev)
    ws = F.Workspace(2048, 8192, device=dev)
    q = F.alloc_layout(2048, 8192, F.SCALE_NV16, device=dev)
    def timed(fn, k):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    def rate(nbytes, n_elem, ms):
        gbps = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 6), "gbps": round(gbps, 1), "elements_per_s": round(n_elem / (ms * 1e-3), 1),
                "frac_of_peak": round(gbps / PEAK_GBPS, 4)}

    sweep = {}
    wn = 2048 * 8192
    for gname, g in (("e1m2", F.GRID_E1M2), ("int4", F.GRID_INT4), ("e2m1", F.GRID_E2M1)):
        for rht in (0, 1):
            c = F.config(g, F.ROUND_RTNE, F.SCALE_NV16, rht=rht, rht_seed=2)
            F.ufp4_quantize(w, c, q, ws, stream)
            st = F.ufp4_stats(w, 0, c, q, ws, stream)
            ms = timed(lambda: F.ufp4_quantize(w, c, q, ws, stream), max(10, steps // 10))
            sweep[f"{gname}_rht{rht}"] = {"sqnr_db": round(st["sqnr_db"], 3),
                                          "mean_signed_err_grid": round(st["mean_signed_err_grid"], 5),
                                          "alpha": round(st["alpha"], 6),
                                          "row_call": rate(2 * wn + wn // 2 + wn // 16 + 4, wn, ms)}
    out["weight_2048x8192_sweep"] = sweep
    del w, ws, q

    for name in ("output_grad_16384x4096_sr", "moe_65536x4096_grouped", "moe_65536x4096_grouped_delayed"):
        fn, nbytes, n_elem, keep = workload_leg(torch, F, synth, np, dev, stream, name)
        out[name] = rate(nbytes, n_elem, timed(fn, max(10, steps // 10)))
        del fn, keep
    # compounding of the GEMM gain: 16 layers, 8192 tokens x 1024, orthogonal weights
    import fp4_quantization_amd.shrinkage as S
    T, D, L = 8192, 1024, 16
    h0 = torch.from_numpy(synth.activation(T, D, seed=21).view(np.int16)).to(dev)
    Ws = [torch.from_numpy(synth.orthogonal(D, seed=100 + i).view(np.int16)).to(dev) for i in range(L)]
    chain = {}
    for gname, gg in (("e1m2", F.GRID_E1M2), ("e2m1", F.GRID_E2M1)):
        for rht in (0, 1):
            r = S.shrinkage_chain(h0, Ws, F.config(gg, F.ROUND_RTNE, F.SCALE_NV16, rht=rht, rht_seed=5), stream)
            eta = np.array(r["eta"])
            chain[f"{gname}_rht{rht}"] = {"mean_eta": round(float(eta.mean()), 6),
                                          "prod_eta": round(float(eta.prod()), 5),
                                          "exp_minus_sum_delta": round(float(np.exp(-(1.0 - eta).sum())), 5),
                                          "chain_gain": round(r["gain"][-1], 5)}
    out["shrinkage_chain_8192x1024_16_layers"] = chain
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the warm figure (repeated calls on one buffer set, input cache-resident)")
    ap.add_argument("--schedule", choices=("auto", "two-pass", "single-pass"), default="auto",
                    help="schedule of the timed calls (the other one is timed beside it)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the legs beyond the headline workload's own (the profiler runs use it: those "
                         "legs launch the same kernels on other tensors)")
    ap.add_argument("--workload", choices=WORKLOADS, default=None,
                    help="profiler runs: time only this workload's call (no headline line)")
    ap.add_argument("--copy", action="store_true",
                    help="time a plain device copy of 512 MiB instead (bandwidth and counter calibration)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                              "COPY_WRITE_DIR"),
                    help="write the counter summary from four rocprofv3 --pmc output directories "
                         "(this run, FETCH_SIZE then WRITE_SIZE; --copy run, the same) and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        d = args.summarize_counters
        run = (f"python3 bench.py --workload {args.workload} --steps 5 --warmup 2" if args.workload else
               "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-extra --no-warm")
        wl = f" --workload {args.workload}" if args.workload else ""
        summarize_counters(*d, workload=args.workload, commands=[
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d[0]} -o run -- {run}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d[1]} -o run -- {run}",
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d[2]} -o run -- "
            "python3 bench.py --copy --steps 5 --warmup 2",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d[3]} -o run -- "
            "python3 bench.py --copy --steps 5 --warmup 2",
            f"python3 bench.py --summarize-counters {' '.join(d)}{wl}"])
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the per-tensor amax exchange a multi-GPU run would need is not built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_quantization_amd as F
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import ctypes

    if args.copy:
        copy_bench(torch, args)
        return
    if args.workload:
        run_workload(torch, F, synth, np, args)
        return

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)  # default priority
    torch.cuda.set_stream(stream)
    xb = synth.activation(ROWS, COLS, seed=1)
    x0 = torch.from_numpy(xb.view(np.int16)).to(dev)
    cfg = F.config(F.GRID_E1M2, F.ROUND_RTNE, F.SCALE_NV16, rht=1, rht_seed=1)
    cfg_off = F.config(F.GRID_E1M2, F.ROUND_RTNE, F.SCALE_NV16, rht=0, rht_seed=1)
    set_bytes = ROWS * COLS * 2 + algorithmic_bytes(ROWS, COLS)
    n_sets = max(12, -(-600_000_000 // set_bytes))
    sets = []
    for _ in range(n_sets):
        sets.append((x0.clone(), F.alloc_layout(ROWS, COLS, F.SCALE_NV16, device=dev),
                     F.alloc_layout(COLS, ROWS, F.SCALE_NV16, device=dev), F.Workspace(ROWS, COLS, device=dev)))
    torch.cuda.synchronize()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def prebuilt(c):
        fns = []
        for x, row, col, ws in sets:
            a = (ctypes.c_void_p(x.data_ptr()), ROWS, COLS, COLS, ctypes.byref(c), row.c(), col.c(),
                 ws.ptr, ws.nbytes, sptr)

            def fn(a=a):
                rc = F.lib.ufp4_quantize_rowcol(*a)
                if rc:
                    raise F.Ufp4Error("ufp4_quantize_rowcol", rc)
            fns.append(fn)
        return fns

    modes = {"auto": F.SCHEDULE_AUTO, "two-pass": F.SCHEDULE_TWO_PASS, "single-pass": F.SCHEDULE_SINGLE_PASS}
    F.ufp4_set_schedule(modes[args.schedule])
    single = F.ufp4_schedule_of(ROWS, COLS, cfg, both_layouts=True) == F.SCHEDULE_SINGLE_PASS
    on, off = prebuilt(cfg), prebuilt(cfg_off)
    ms, graph = time_graph(torch, on, args.steps, args.warmup, stream)
    ms_off, _ = time_graph(torch, off, args.steps, args.warmup, stream)
    ms_eager = time_eager(torch, on, args.steps, args.warmup, stream)
    ms_warm = None if args.no_warm else time_graph(torch, on[:1], args.steps, args.warmup, stream)[0]
    # bandwidth reference: the same loads and output bytes with no arithmetic
    roof_fns = []
    for x, row, col, ws in sets:
        ra = (ctypes.c_void_p(x.data_ptr()), ROWS, COLS, row.c(), col.c(), sptr)

        def rfn(a=ra):
            rc = F.lib.ufp4_roof_rowcol(*a)
            if rc:
                raise F.Ufp4Error("ufp4_roof_rowcol", rc)
        roof_fns.append(rfn)
    ms_roof, _ = time_graph(torch, roof_fns, args.steps, args.warmup, stream)
    # per-kernel durations: hipEvents around each kernel of one call, on the
    # launch stream, over calls that rotate through the buffer sets
    per_kernel = []
    for i in range(args.steps):
        x, row, col, ws = sets[i % len(sets)]
        per_kernel.append(F.ufp4_time_rowcol(x, cfg, row, col, ws, stream))
    k_amax = np.array([a for a, _ in per_kernel])
    k_quant = np.array([b for _, b in per_kernel])
    # delayed scaling (a different numerics mode, reported beside, never as
    # the value): each call reads the previous call's tile maxima
    n_amax = F.ufp4_amax_tiles(ROWS, COLS)
    amax = [torch.tensor([[3.0, 5.0]], dtype=torch.float32, device=dev).repeat(n_amax, 1) for _ in sets]
    dfns = []
    for i, (x, row, col, ws) in enumerate(sets):
        a = (ctypes.c_void_p(x.data_ptr()), ROWS, COLS, COLS, ctypes.byref(cfg),
             ctypes.c_void_p(amax[i - 1].data_ptr()), n_amax, ctypes.c_void_p(amax[i].data_ptr()),
             row.c(), col.c(), sptr)

        def dfn(a=a):
            rc = F.lib.ufp4_quantize_delayed(*a)
            if rc:
                raise F.Ufp4Error("ufp4_quantize_delayed", rc)
        dfns.append(dfn)
    ms_delayed, _ = time_graph(torch, dfns, args.steps - args.steps % len(sets) or len(sets), args.warmup, stream)
    # consumer GEMM (reported beside): the activation's row-wise codes times a
    # quantized 8192 x 2048 weight's, C = X W^T of 8192 x 8192 (fwd_y), K = 2048
    wq = F.alloc_layout(ROWS, COLS, F.SCALE_NV16, device=dev)
    wx = torch.from_numpy(synth.weight(ROWS, COLS, seed=2).view(np.int16)).to(dev)
    F.ufp4_quantize(wx, cfg, wq, sets[0][3])
    gc = torch.empty((ROWS, ROWS), dtype=torch.float32, device=dev)
    xq = sets[0][1]
    gemm_fns = [lambda: F.ufp4_gemm_nt(cfg, xq, wq, ROWS, ROWS, COLS, gc, stream)]
    gemm_steps = 20
    ms_gemm, _ = time_graph(torch, gemm_fns, gemm_steps, 3, stream)
    gemm_tflops = 2.0 * ROWS * ROWS * COLS / (ms_gemm * 1e-3) / 1e12
    # the same product with MX32 operands on the scaled f8f6f4 MFMA: E2M1
    # codes as FP4 (peak 10.1 PFLOP/s), E1M2 codes expanded to FP8 (5.0)
    mx_gemm = {}
    for gname, g, peak in (("e2m1_fp4", F.GRID_E2M1, 10100.0), ("e1m2_fp8", F.GRID_E1M2, 5000.0)):
        cm = F.config(g, F.ROUND_RTNE, F.SCALE_MX32, rht=1, rht_seed=1)
        xm = F.alloc_layout(ROWS, COLS, F.SCALE_MX32, device=dev)
        wm = F.alloc_layout(ROWS, COLS, F.SCALE_MX32, device=dev)
        F.ufp4_quantize(x0, cm, xm, sets[0][3])
        F.ufp4_quantize(wx, cm, wm, sets[0][3])
        ms_m, _ = time_graph(torch, [lambda: F.ufp4_gemm_nt(cm, xm, wm, ROWS, ROWS, COLS, gc, stream)],
                             gemm_steps, 3, stream)
        tf = 2.0 * ROWS * ROWS * COLS / (ms_m * 1e-3) / 1e12
        mx_gemm[f"gemm_mx32_{gname}"] = {"ms": round(ms_m, 6), "tflops": round(tf, 1),
                                         "frac_of_peak": round(tf / peak, 4)}
        del xm, wm
    del gc
    # the other schedule on the same buffers, for comparison
    other = "two_pass" if single else "single_pass"
    F.ufp4_set_schedule(F.SCHEDULE_TWO_PASS if single else F.SCHEDULE_SINGLE_PASS)
    ms_other, _ = time_graph(torch, on, args.steps, args.warmup, stream)
    tk = []
    for i in range(args.steps):
        x, row, col, ws = sets[i % len(sets)]
        tk.append(F.ufp4_time_rowcol(x, cfg, row, col, ws, stream))
    two = {f"{other}_ms": round(ms_other, 6),
           f"{other}_quant_kernel_ms_mean": round(float(np.mean([b for _, b in tk])), 6),
           f"{other}_time_ratio": round(ms_other / ms, 4)}
    if other == "two_pass":  # the single pass has no maxima kernel to time
        two[f"{other}_amax_kernel_ms_mean"] = round(float(np.mean([a for a, _ in tk])), 6)
    F.ufp4_set_schedule(modes[args.schedule])
    # the graph's outputs equal an eager call's
    x, row, col, ws = sets[0]
    ref_row, ref_col = row.codes.clone(), col.codes.clone()
    row.codes.zero_()
    col.codes.zero_()
    on[0]()
    torch.cuda.synchronize()
    assert torch.equal(ref_row, row.codes) and torch.equal(ref_col, col.codes), "graph replay != eager call"

    nbytes = algorithmic_bytes(ROWS, COLS)
    gbps = nbytes / (ms * 1e-3) / 1e9
    traffic_quant, traffic_call = counter_traffic(single)
    quant_gbps = nbytes / (float(k_quant.mean()) * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "activation 8192x2048 bf16, N(0,1) + channel bias N(0,0.5), 2 channels x50; "
                               "RHT (seed 1) + E1M2 RTNE, E4M3 per-16 + FP32 per-tensor scales, row+col",
                   "rows": ROWS, "cols": COLS, "buffer_sets": n_sets,
                   "algorithmic_bytes_per_call": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(quant_gbps, 2), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(quant_gbps / PEAK_GBPS, 4), "traffic": traffic_quant,
                     "kernel": ("ufp4_single_kernel<E1M2, RTNE, RHT> (single pass, the whole call)" if single
                                else "ufp4_quant_kernel<E1M2, RTNE, NV16, RHT>"),
                     "bytes_per_launch": nbytes,
                     "kernel_ms_mean": round(float(k_quant.mean()), 6),
                     # the measured rate of the same loads and output bytes
                     # with no arithmetic (ufp4_roof_rowcol), and the
                     # kernel's fraction of it
                     "attainable_gbps": round(nbytes / (ms_roof * 1e-3) / 1e9, 1),
                     "frac_of_attainable": round(quant_gbps / (nbytes / (ms_roof * 1e-3) / 1e9), 4)},
        "extra": {"elements_per_s": round(ROWS * COLS / (ms * 1e-3), 1),
                  "call_frac_of_peak": round(gbps / PEAK_GBPS, 4),
                  "call_hbm_bytes_counted": traffic_call,
                  "quant_kernel_ms_median": round(float(np.median(k_quant)), 6),
                  "event_call_ms_median": round(float(np.median(k_amax + k_quant)), 6),
                  "roof_ms": round(ms_roof, 6),
                  "roof_gbps": round(nbytes / (ms_roof * 1e-3) / 1e9, 1),
                  "call_time_over_roof": round(ms / ms_roof, 4),
                  "rht_off_ms": round(ms_off, 6),
                  "rht_overhead": round(ms / ms_off - 1.0, 4),
                  "eager_launch_ms": round(ms_eager, 6),
                  "schedule": "single-pass" if single else "two-pass",
                  "timing": "HIP graph of the K calls, one replay, hipEvents on the launch stream"},
    }
    if not single:  # the single pass has no maxima kernel to time
        line["extra"]["amax_kernel_ms_mean"] = round(float(k_amax.mean()), 6)
        line["extra"]["amax_kernel_ms_median"] = round(float(np.median(k_amax)), 6)
    if two:
        line["extra"].update(two)
    line["extra"]["gemm_8192x8192x2048_ms"] = round(ms_gemm, 6)
    line["extra"]["gemm_tflops"] = round(gemm_tflops, 1)
    line["extra"]["gemm_frac_of_fp16_mfma_peak"] = round(gemm_tflops / 2500.0, 4)
    line["extra"].update(mx_gemm)
    line["extra"]["delayed_scaling_ms"] = round(ms_delayed, 6)
    line["extra"]["delayed_scaling_gbps"] = round(nbytes / (ms_delayed * 1e-3) / 1e9, 2)
    if ms_warm is not None:
        line["extra"]["warm_same_buffer_ms"] = round(ms_warm, 6)
        line["extra"]["warm_same_buffer_gbps"] = round(nbytes / (ms_warm * 1e-3) / 1e9, 2)
    if not args.no_extra:
        line["extra"].update(variant_legs(torch, F, sets, stream, args.steps))
        line["extra"].update(extra_legs(torch, F, synth, np, dev, stream, args.steps))
        line["extra"]["call_frac_of_copy"] = round(gbps / line["extra"]["copy_gbps"], 4)
        line["extra"]["quant_kernel_frac_of_copy"] = round(quant_gbps / line["extra"]["copy_gbps"], 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(xb)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
