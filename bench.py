#!/usr/bin/env python3
"""Benchmark of the register-tile GEMM on one MI355X.

A step is one call of the whole hot path -- validation, tile selection and
the single fused GEMM kernel -- on the workload's operands, already resident
in HBM.  The default workload is the 4096^3 fp16 GEMM (fp32 accumulation,
fp16 output) with inputs N(0,1)/8.

Order of a run: the real-time counter's rate (one long clock probe timed
with events); the yardsticks -- the streaming read, then the matrix-core-only
loop for about --settle-ms (which also brings the part from its idle clock
to its loaded one); --warmup untimed steps; a clock probe; exactly --steps
steps timed back to back between two HIP events on the launch stream; a
clock probe; the oracle on the host.  Prints ONE JSON line:

  value        whole-job TFLOP/s = 2*M*N*K / mean step time of the timed region
  roofline     the GEMM kernel against the dense fp16 matrix-core peak
               (2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096 FLOP/clk), or for
               the M <= 16 workload against the 8 TB/s HBM peak, from the
               same timed region (a step is one kernel launch); the shader
               clock right before and right after it; its HBM GB/s; the
               yardsticks' rates (context); and, when the committed rocprofv3
               counters were taken on the current kernel source, the HBM
               traffic and matrix-core figures from those counters, with
               where they were taken
  cpu_baseline the oracle (plain fp64 C, all host cores) timed on a bounded
               row sample of the same workload, scaled to TFLOP/s, and its
               one-core rate on a slice of it
  parity       the GPU result on the same sampled rows against the oracle
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (fp16→fp32 acc) at 4096³ + % of MFMA peak (rocprof)"
PEAK_TFLOPS = {1: 2516.6, 2: 2516.6, 3: 157.3}   # dense f16 / bf16 / f32 matrix-core peak
PEAK_HBM_GBS = 8000.0
# fp32 fused multiply-add on the vector lanes, one per lane per cycle (the
# library is built without packed fp32): 256 CUs x 4 SIMDs x 16 lanes x 2
# FLOP x 2.4 GHz
PEAK_VALU_F32_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
WORKLOADS = ("square", "epilogue", "ragged", "skinny", "f32square", "regtile")


def _code_tokens(src):
    """C++ source without its comments, whitespace runs collapsed: what the
    compiler sees, so that editing a comment does not orphan the counters."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def cpu_model():
    """The host CPU's model name (for the oracle baseline), or "" if unknown."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def device_info():
    """The GPU the run used: name, architecture, compute units, memory."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", ""),
            "compute_units": pr.multi_processor_count,
            "L2_MiB_per_XCD": round(getattr(pr, "L2_cache_size", 0) / 2 ** 20, 1),
            "memory_GiB": round(pr.total_memory / 2 ** 30, 1)}


def csrc_digest():
    """Digest of the kernel sources (comments aside) and the compile flags."""
    from thread_register_tile_amd import build
    h = hashlib.sha256()
    d = os.path.join(ROOT, "thread_register_tile_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_tokens(f.read()).encode())
    h.update(repr((build.FLAGS, build.FILE_FLAGS)).encode())
    return h.hexdigest()[:16]


def committed_counters(workload):
    """Counter figures of `workload` from profiles/counters.json, only if they
    were taken on the current kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("csrc_digest") != csrc_digest():
        return None
    return e


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def _step_kernel(name):
    """Whether a kernel is part of a GEMM step: the GEMM kernel itself, or the
    reduction that completes the split-K streaming path."""
    return "gemm" in name or "skinny_split_reduce" in name


def _per_step(rows, value):
    """A step's figure: the median over the launches of each of the step's
    kernels, summed over those kernels (one for most workloads, two for the
    split-K path)."""
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(value(r))
    return sum(_median(v) for v in by.values())


def ingest_counters(root):
    """Build profiles/counters.json from rocprofv3 --pmc runs of this script.

    root/pmc_fetch_<w>, root/pmc_write_<w>: FETCH_SIZE and WRITE_SIZE runs with
    --copy-calibration-mib 256; root/pmc_mfma_<w>: SQ_INSTS_VALU_MFMA_MOPS_*,
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE and
    SQ_LDS_BANK_CONFLICT.  Each counter is scaled by what it reads for the
    256 MiB device-to-device copy of the same run (read and written bytes
    known), and the GEMM launches' median is kept.  root/provenance.json, if
    present, is stored with every workload's figures."""
    import workloads as W
    out = {}
    # where and how the counters were taken: root/provenance.json, written
    # by whoever ran the profiler (date, GPU, commands), kept with the figures
    prov = {}
    try:
        with open(os.path.join(root, "provenance.json")) as f:
            prov = json.load(f)
    except (OSError, ValueError):
        pass
    for w in WORKLOADS:
        cfg = W.CONFIGS[w]
        e = {"csrc_digest": csrc_digest(), "provenance": prov}
        for cn, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
            path = os.path.join(root, f"pmc_{cn}_{w}", "run_counter_collection.csv")
            if not os.path.exists(path):
                break
            rows = [r for r in _csv_rows(path) if r["Counter_Name"] == counter]
            copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
            big = max(int(r["Grid_Size"]) for r in copies)
            raw_copy = float(next(r["Counter_Value"] for r in copies if int(r["Grid_Size"]) == big))
            gemm = [r for r in rows if _step_kernel(r["Kernel_Name"])]
            raw = _per_step(gemm, lambda r: float(r["Counter_Value"]))
            factor = 256 * 1024 / raw_copy
            e["kernel"] = " + ".join(sorted({r["Kernel_Name"] for r in gemm}))
            e[f"{cn}_size_kib_raw"] = raw
            e[f"{cn}_factor"] = round(factor, 5)
            e[f"{cn}_bytes_per_launch"] = int(raw * 1024 * factor)
        if "write_bytes_per_launch" in e:
            e["bytes_per_launch"] = e["fetch_bytes_per_launch"] + e["write_bytes_per_launch"]
        path = os.path.join(root, f"pmc_mfma_{w}", "run_counter_collection.csv")
        if os.path.exists(path):
            rows = [r for r in _csv_rows(path) if _step_kernel(r["Kernel_Name"])]
            med = {c: _per_step([r for r in rows if r["Counter_Name"] == c],
                                lambda r: float(r["Counter_Value"]))
                   for c in sorted({r["Counter_Name"] for r in rows})}
            first = rows[0]["Counter_Name"]
            ns = _per_step([r for r in rows if r["Counter_Name"] == first],
                           lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            mops = sum(v for k, v in med.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
            gui = med.get("GRBM_GUI_ACTIVE", 0.0) / 8          # summed over the 8 XCDs
            busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            e["mfma"] = {"counters": med, "duration_ns": ns,
                         "flops_per_launch": mops * 512, "flops_algorithmic": cfg.flops,
                         "tflops": round(mops * 512 / ns / 1e3, 2),
                         "frac_of_peak": round(mops * 512 / ns / 1e3 / PEAK_TFLOPS[cfg.dtype], 4),
                         "clock_ghz": round(gui / ns, 3) if gui else None,
                         "busy_frac": round(busy / (gui * 1024), 4) if gui else None}
        out[w] = e
    with open(COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def stream_read_gbps(trt, torch, nbytes=1 << 30, reps=20, settle_ms=0.0):
    """Read bandwidth of the library's plain streaming-read kernel over a
    buffer larger than the last-level cache: `reps` launches timed back to
    back with events, after enough untimed ones to fill settle_ms."""
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(trt.READ_PROBE_SINK_BYTES, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(max(5, int(settle_ms / 0.17))):       # ~0.17 ms per 1 GiB read
        trt.hbm_read_probe(x, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        trt.hbm_read_probe(x, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / reps * 1e-3
    del x
    return nbytes / s / 1e9


def mfma_loop_tflops(trt, torch, host_a, dtype, run_ms, launch_ms=0.1, reps=20):
    """Rate of the library's matrix-core-only loop on operand words taken from
    the workload's own A data: launches of about launch_ms each, back to back
    for about run_ms in all; the last `reps` are timed with events."""
    import numpy as np
    words = np.resize(host_a, trt.MFMA_PROBE_OPERAND_BYTES // host_a.itemsize)  # repeats a short input
    ops = torch.from_numpy(words.view(np.int8)).cuda()
    sink = torch.empty(trt.MFMA_PROBE_SINK_BYTES // 4, dtype=torch.float32, device="cuda")
    iters = max(1, int(launch_ms * 1e-3 * 1.8e9 / (32 * 32)))   # 32 products of 32 cycles per round
    stream = torch.cuda.current_stream()
    for _ in range(max(0, int(run_ms / launch_ms) - reps)):
        trt.mfma_loop_probe(ops, iters, dtype, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        trt.mfma_loop_probe(ops, iters, dtype, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / reps * 1e-3
    return trt.mfma_loop_probe_flops(iters, dtype) / s / 1e12


class Clock:
    """Shader clock from the library's clock probe (cycles over real-time
    ticks).  The real-time counter's rate is measured once, by timing a long
    probe with events; each reading is a short probe enqueued on the current
    stream, read back after the next synchronisation."""

    def __init__(self, trt, torch):
        self.trt, self.torch = trt, torch
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ticks = 200_000
        trt.clock_probe(ticks)                      # first launch: not timed
        e0.record(s)
        out = trt.clock_probe(ticks)
        e1.record(s)
        torch.cuda.synchronize()
        self.rt_hz = float(out[:, 1].float().median().item()) / (e0.elapsed_time(e1) * 1e-3)
        self.pending = {}

    def mark(self, name, ticks=2000):
        """Enqueue a reading of about ticks / rt_hz seconds (20 us at 100 MHz)."""
        self.pending[name] = self.trt.clock_probe(ticks)

    def ghz(self, name):
        c = self.pending[name].cpu().numpy()
        return round(float((c[:, 0] / c[:, 1]).mean()) * self.rt_hz / 1e9, 3)


def counters_entry(counters):
    """Where the committed counter figures came from."""
    return {"file": "profiles/counters.json", "csrc_digest": counters.get("csrc_digest"),
            **counters.get("provenance", {})}


def bench_reduce(args, trt, torch, np, W):
    """The rank-1 block reduction workload: one JSON line in HBM GB/s."""
    from oracle import reduce_ref as RR
    w = W.REDUCE
    bits = W.make_reduce_input(w)
    x = torch.from_numpy(bits.view(np.int32 if bits.dtype == np.uint32 else np.int16)).cuda()
    out = torch.empty(w.nblocks, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def step():
        trt.block_reduce_raw(x.data_ptr(), w.n, w.block, w.dtype, w.op, out.data_ptr(), sptr)

    # the streaming-read yardstick first, for about --settle-ms (see main())
    sr = None if args.no_stream_read else stream_read_gbps(trt, torch, settle_ms=args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                "algorithmic_bytes": w.algorithmic_bytes, "kernel_ms": round(ms, 5),
                "timing": f"mean of {args.steps} back-to-back launches between HIP events "
                          "on the launch stream (the timed region)"}
    if sr is not None:
        roofline["stream_read_GBps"] = round(sr, 1)
        roofline["frac_of_stream_read"] = round(gbs / sr, 4)
    cpu = parity = None
    if not args.no_cpu_baseline:
        got = out.cpu().numpy()
        # the oracle on the first blocks, sized to the CPU budget by a short run
        t0 = time.perf_counter()
        RR.block_reduce(bits[:64 * w.block], w.dtype, 64 * w.block, w.block, w.op)
        per_block = (time.perf_counter() - t0) / 64
        nb = int(min(w.nblocks, max(64, args.cpu_seconds / max(per_block, 1e-9))))
        t0 = time.perf_counter()
        ref = RR.block_reduce(bits[:nb * w.block], w.dtype, nb * w.block, w.block, w.op)
        t_cpu = time.perf_counter() - t0
        cpu = {"value": (W.ELEM_BYTES[w.dtype] * nb * w.block + 4 * nb) / t_cpu / 1e9,
               "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"blocks 0..{nb - 1} of {w.nblocks} (python + fsum, one core), {t_cpu:.1f} s",
               "cpu_model": cpu_model()}
        import oracle
        err = np.abs(got[:nb].astype(np.float64) - ref)
        absum = np.abs(oracle.decode(bits[:nb * w.block], w.dtype)).reshape(nb, w.block).sum(1)
        bound = w.block * 2.0 ** -24 * absum + 2.0 ** -24 * np.abs(ref)   # binary32 summation
        parity = {"blocks": nb, "max_abs": float(err.max()), "ok": bool((err <= bound).all())}
    line = {
        "metric": "rank-1 block reduction, HBM GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": W.DTYPE_NAMES[w.dtype],
        "data": "synthetic",
        "config": {"workload": f"block sum of {w.n} f16 elements, BLOCK={w.block}",
                   "n": w.n, "block": w.block, "op": ["sum", "max", "min"][w.op],
                   "csrc_digest": csrc_digest()},
        "roofline": roofline, "cpu_baseline": cpu, "parity": parity, "device": device_info(),
    }
    print(json.dumps(line), flush=True)


def oracle_rows(oracle, w, host, rows, threads, n_range=None):
    """The oracle on rows 0..rows-1 (and n_range) of workload w; (result, seconds)."""
    t0 = time.perf_counter()
    ref = oracle.gemm_block(w.M, w.N, w.K, host["A"], w.lda_, w.opA, host["B"], w.ldb_, w.opB,
                            w.dtype, bias=host["bias"], relu=w.relu, R=host["R"],
                            ldr=w.ldr_ if host["R"] is not None else 0, out_dtype=w.odt,
                            scale=host["scale"], m_range=(0, rows), n_range=n_range,
                            threads=threads)
    return ref, time.perf_counter() - t0


def cpu_baseline(args, w, host, C, np):
    """The oracle timed on the host cores: a row sample of the workload sized
    to about --cpu-seconds on all cores the process may use, plus a one-core
    rate on a slice of it; the sample also serves as the run's parity check."""
    import oracle
    threads = oracle.default_threads()
    # calibrate: the per-call cost (decoding B once) and the per-row cost,
    # from two short runs; then size the sample to the budget
    r1, r2 = min(threads, w.M), min(4 * threads, w.M)
    t1 = oracle_rows(oracle, w, host, r1, threads)[1]
    t2 = oracle_rows(oracle, w, host, r2, threads)[1]
    per_row = max((t2 - t1) / max(r2 - r1, 1), 1e-6)
    fixed = max(t1 - r1 * per_row, 0.0)
    rows = int(min(w.M, max(r1, (args.cpu_seconds - fixed) / per_row)))
    rows = max(1, rows - rows % max(1, min(threads, rows)))
    ref, t_cpu = oracle_rows(oracle, w, host, rows, threads)
    # one core: the first rows (at most 64) over at most 1024 columns
    r1c, n1c = min(64, w.M), min(1024, w.N)
    t_1 = oracle_rows(oracle, w, host, r1c, 1, n_range=(0, n1c))[1]
    cpu = {"value": 2.0 * rows * w.N * w.K / t_cpu / 1e12, "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": f"rows 0..{rows - 1} of C ({rows}x{w.N}x{w.K}, fp64 oracle incl. "
                     f"epilogue), {t_cpu:.1f} s on {threads} threads",
           "per_core": {"value": 2.0 * r1c * n1c * w.K / t_1 / 1e12, "unit": "TFLOP/s",
                        "sample": f"rows 0..{r1c - 1}, columns 0..{n1c - 1}, one thread, "
                                  f"{t_1:.2f} s"},
           "cpu_model": cpu_model()}
    out_bytes = W_ELEM_BYTES[w.odt]
    Cg = C.cpu().numpy().view(np.uint32 if out_bytes == 4 else np.uint16)
    Cg = Cg.reshape(w.M, w.ldc_)[:rows, :w.N]
    rep = oracle.accept(np.ascontiguousarray(Cg), ref, w.odt)
    parity = {"rows": rows, "ok": rep["ok"], "max_abs": rep["max_abs"],
              "frob_rel": rep["frob_rel"], "bit_match": rep["bit_match"]}
    return cpu, parity


W_ELEM_BYTES = {1: 2, 2: 2, 3: 4}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="square")
    ap.add_argument("--tile", default=None, help="BM,BN,BK")
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="wall time of the yardsticks run before the GEMM (the part leaves "
                         "its idle clock over the first ~20 ms of load)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB before the "
                         "GEMM steps (a known-size kernel to scale HBM counters by)")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the streaming-read bandwidth measurement")
    ap.add_argument("--no-mfma-loop", action="store_true",
                    help="skip the matrix-core-only loop measurement")
    ap.add_argument("--no-workspace", action="store_true",
                    help="call trt_gemm (no workspace) even where trt_gemm_ws would split K")
    ap.add_argument("--ingest-counters", metavar="DIR", default=None,
                    help="write profiles/counters.json from rocprofv3 --pmc runs in DIR "
                         "and exit (no GPU needed)")
    args = ap.parse_args()

    if args.ingest_counters:
        print(json.dumps(ingest_counters(args.ingest_counters), indent=1))
        return

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for {args.gpus}); "
              "the path has no multi-GPU sharding.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import thread_register_tile_amd as trt
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    trt.lib()  # fail loudly if the HIP library is missing

    if args.workload == "reduce":
        return bench_reduce(args, trt, torch, np, W)
    w = W.CONFIGS[args.workload]
    tile = tuple(int(x) for x in args.tile.split(",")) if args.tile else w.tile
    host = W.make_inputs(w)
    dev = lambda b: None if b is None else torch.from_numpy(
        b.view(np.int32 if b.dtype == np.uint32 else np.int16)).cuda()
    A, B, bias, R = dev(host["A"]), dev(host["B"]), dev(host["bias"]), dev(host["R"])
    scale = dev(host["scale"])
    out_bytes = W.ELEM_BYTES[w.odt]
    C = torch.empty(w.M * w.ldc_, dtype=torch.int32 if out_bytes == 4 else torch.int16,
                    device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    mfma_bound = w.name != "skinny" and w.regtile is None

    def step_regtile():
        lm, ln, mt = w.regtile
        trt.gemm_regtile_raw(w.M, w.N, w.K, A.data_ptr(), w.lda_, w.opA, B.data_ptr(), w.ldb_,
                             w.opB, C.data_ptr(), w.ldc_, w.dtype, w.odt, lm, ln, mt,
                             bias=bias.data_ptr() if bias is not None else 0, relu=w.relu,
                             residual=R.data_ptr() if R is not None else 0,
                             ldr=w.ldr_ if R is not None else 0,
                             scale=scale.data_ptr() if scale is not None else 0, stream=sptr)

    # shapes that split K over workgroups (M <= 16) run through trt_gemm_ws,
    # with the workspace allocated here, before any timing
    ws_bytes = 0 if (w.regtile is not None or tile is not None or args.no_workspace) else \
        trt.workspace_size(w.M, w.N, w.K, w.opA, w.opB, w.dtype)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda") if ws_bytes else None

    def step():
        if w.regtile is not None:
            return step_regtile()
        kw = dict(bias=bias.data_ptr() if bias is not None else 0, relu=w.relu,
                  residual=R.data_ptr() if R is not None else 0,
                  ldr=w.ldr_ if R is not None else 0,
                  scale=scale.data_ptr() if scale is not None else 0, stream=sptr)
        if ws is not None:
            return trt.gemm_ws_raw(w.M, w.N, w.K, A.data_ptr(), w.lda_, w.opA, B.data_ptr(),
                                   w.ldb_, w.opB, C.data_ptr(), w.ldc_, w.dtype, w.odt,
                                   workspace=ws.data_ptr(), workspace_bytes=ws_bytes, **kw)
        trt.gemm_raw(w.M, w.N, w.K, A.data_ptr(), w.lda_, w.opA, B.data_ptr(), w.ldb_, w.opB,
                     C.data_ptr(), w.ldc_, w.dtype, w.odt, tile=tile, **kw)

    clock = Clock(trt, torch)

    # The yardsticks first: the streaming read (HBM context), then the
    # matrix-core-only loop on the workload's own A data for about
    # --settle-ms.  Besides their rates, they take the part out of its idle
    # clock state, so that the GEMM below is timed under load, as the
    # yardstick is; the clock probes record the clock around the timed region.
    roofline_ctx = {}
    if not args.no_stream_read:
        sr = stream_read_gbps(trt, torch, settle_ms=0.0 if mfma_bound else args.settle_ms)
        roofline_ctx["stream_read_GBps"] = round(sr, 1)
    if mfma_bound and not args.no_mfma_loop:
        a_rows = host["A"].reshape(-1)[:w.a_cols] if w.lda_ < w.a_cols else \
            host["A"].reshape(w.a_rows, w.lda_)[:, :w.a_cols].reshape(-1)   # no padding
        roofline_ctx["mfma_loop_tflops"] = round(
            mfma_loop_tflops(trt, torch, a_rows, w.dtype, args.settle_ms), 1)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    clock.mark("before")
    torch.cuda.synchronize()

    # timed region: events on the launch stream bracket exactly `steps` calls
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    clock.mark("after")
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    # A step is one launch of one kernel, enqueued back to back: the timed
    # region's mean per launch is the kernel's average duration plus the
    # gap between launches (a few microseconds), so value and roofline
    # share one timing.
    tflops = w.flops / (ms * 1e-3) / 1e12
    counters = committed_counters(w.name)
    traffic = counters.get("bytes_per_launch") if counters else None
    roofline = {"bound": "mfma", "achieved": round(tflops, 2),
                "peak": PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                "frac": round(tflops / PEAK_TFLOPS[w.dtype], 4),
                "traffic": traffic,
                "algorithmic_bytes": w.algorithmic_bytes,
                "algorithmic_flops": w.flops,
                "timing": f"mean of {args.steps} back-to-back launches between HIP events "
                          "on the launch stream (the timed region)",
                "kernel_ms": round(ms, 5),
                "clock_ghz": {"before": clock.ghz("before"), "after": clock.ghz("after"),
                              "realtime_counter_MHz": round(clock.rt_hz / 1e6, 2),
                              "probe": "one wave per compute unit, 20 us, enqueued right "
                                       "before and right after the timed region; a light "
                                       "load, so it reads the clock the part offers, "
                                       "which its matrix cores lower under load"},
                "hbm_GBps_algorithmic": round(w.algorithmic_bytes / (ms * 1e-3) / 1e9, 1)}
    if traffic:
        roofline["hbm_GBps_traffic"] = round(traffic / (ms * 1e-3) / 1e9, 1)
        roofline["traffic_source"] = counters_entry(counters)
    if w.name == "skinny":
        gbs = w.algorithmic_bytes / (ms * 1e-3) / 1e9
        roofline.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "tflops": round(tflops, 2)})
    if w.regtile is not None:
        roofline.update({"bound": "alu", "peak": round(PEAK_VALU_F32_TFLOPS, 1),
                         "frac": round(tflops / PEAK_VALU_F32_TFLOPS, 4),
                         "regtile": {"lm": w.regtile[0], "ln": w.regtile[1],
                                     "thread_shape": trt.regtile_thread_shape(*w.regtile)}})
    if counters and "mfma" in counters:
        m = counters["mfma"]
        roofline["rocprof_mfma_committed"] = {
            "tflops": m["tflops"], "frac_of_peak": m["frac_of_peak"],
            "busy_frac": m["busy_frac"], "clock_ghz": m["clock_ghz"],
            "flops_counted": m["flops_per_launch"], "source": counters_entry(counters)}
    roofline.update(roofline_ctx)
    if "mfma_loop_tflops" in roofline_ctx:
        roofline["frac_of_mfma_loop"] = round(tflops / roofline_ctx["mfma_loop_tflops"], 4)
    if w.name == "skinny" and "stream_read_GBps" in roofline_ctx:
        roofline["frac_of_stream_read"] = round(roofline["achieved"] /
                                                roofline_ctx["stream_read_GBps"], 4)

    cpu = parity = None
    if not args.no_cpu_baseline:
        cpu, parity = cpu_baseline(args, w, host, C, np)

    name = {"square": "square 4096x4096x4096 f16 -> f16, fp32 accumulate"}.get(
        w.name, f"{w.name} {w.M}x{w.N}x{w.K}")
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.DTYPE_NAMES[w.dtype],
        "data": "synthetic",
        "config": {"workload": name, "M": w.M, "N": w.N, "K": w.K, "opA": w.opA,
                   "opB": w.opB, "lda": w.lda_, "ldb": w.ldb_, "ldc": w.ldc_,
                   "out_dtype": W.DTYPE_NAMES[w.odt],
                   "epilogue": {"bias": w.bias, "relu": w.relu, "residual": w.residual,
                                "row_scale": w.row_scale},
                   "tile": (f"vector-lane register tile {w.regtile[0]}x{w.regtile[1]}" if w.regtile
                            else list(tile) if tile else "auto"),
                   "settle_ms": args.settle_ms,
                   "entry_point": "trt_gemm_ws (split K, workspace of %d bytes)" % ws_bytes
                   if ws is not None else ("trt_gemm_regtile" if w.regtile is not None
                                           else "trt_gemm_tiled"),
                   "csrc_digest": csrc_digest()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "device": device_info(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
