#!/usr/bin/env python3
"""Benchmark of the fp16 GEMM / M=1 decode GEMV hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs
resident in HBM: gemm_f16 (pick_tile + MFMA kernel) on every square size of
the measured range, 256^3 through 8192^3, then gemm_f16 at M=1, K=4096,
N=12288 (routed to the streaming GEMV) on the next of 8 rotating weight
buffers.  The printed value is the step's algorithmic fp16 FLOP rate.

Before any number is printed the outputs are checked against the CPU oracle
(every element of every square product up to 4096^3, the whole rows of the
8192^3 product that the CPU baseline computes, every element of all 8 decode
products, each output NaN-filled first); a failure prints no throughput.  The dominant kernel (8192^3) and
the GEMV are additionally timed launch by launch with HIP events inside the
timed region, which feed the roofline object.  Per-size, K-sweep and
cold-cache decode details follow the protocol of the pages: warm-up, then
10 repeats, min/median/max.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("fp16 GEMM TFLOP/s (and % MFMA peak) 256³–8192³; "
          "M=1 GEMV µs + HBM GB/s")
# MI355X nominal peaks: 256 CUs x 4096 fp16 FLOP/clk/CU x 2.4 GHz; HBM3E 8 TB/s.
PEAK_FP16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
PEAK_HBM_GBS = 8000.0
SIZES = (256, 512, 768, 1024, 1536, 2048, 4096, 8192)
# seed index of each size's operands (matches the parity tests)
SEED_INDEX = {256: 0, 512: 1, 768: 1, 1024: 1, 1536: 1, 2048: 1, 4096: 2, 8192: 2}
DOMINANT = 8192


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # about 10 s of steps: the clock and power settle over seconds of this load
    ap.add_argument("--warmup", type=int, default=10000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--profile", default=None, metavar="KERNEL",
                    help="instead of the benchmark, launch one kernel repeatedly for a "
                         "profiler: gemm<N> (N^3, e.g. gemm8192), gemv (decode, rotating "
                         "buffers), gemvkn (decode with the weights as K rows of N) or "
                         "copy<MB> (a plain device copy, for counter scaling)")
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--tile", type=int, default=-1)
    ap.add_argument("--variant", type=int, default=-1, help="profile mode: GEMV variant")
    ap.add_argument("--stagger", type=int, default=-1, help="profile mode: -1 the plan's choice, 0 off, 1 on")
    return ap.parse_args()


def profile_mode(args):
    """Repeated launches of one kernel, no oracle and no timing: the workload a
    rocprofv3 kernel-trace or counter pass is taken on."""
    import torch

    from shape_driven_tile_amd import binding as sdt
    from shape_driven_tile_amd import inputs
    dev = torch.device("cuda:0")
    name = args.profile
    if name.startswith("gemm"):
        n = int(name[4:])
        A, B = inputs.square_operands(n, SEED_INDEX.get(n, 2))
        dA = torch.from_numpy(A).to(dev)
        dB = torch.from_numpy(B).to(dev)
        C = torch.empty((n, n), dtype=torch.float16, device=dev)
        for _ in range(args.launches):
            sdt.gemm_f16_ex(dA, dB, C, tile_id=args.tile, stagger=args.stagger)
    elif name == "gemv":
        x = torch.from_numpy(inputs.decode_activations()).to(dev)
        Ws = [torch.from_numpy(inputs.decode_weights(r)).to(dev)
              for r in range(inputs.DECODE_BUFFERS)]
        y = torch.empty((inputs.DECODE_N,), dtype=torch.float16, device=dev)
        for j in range(args.launches):
            sdt.gemv_f16_m1(x, Ws[j % len(Ws)], y)
    elif name == "gemvkn":
        x = torch.from_numpy(inputs.decode_activations()).to(dev)
        Ws = [torch.from_numpy(inputs.decode_weights_kn(r)).to(dev)
              for r in range(inputs.DECODE_BUFFERS)]
        y = torch.empty((inputs.DECODE_N,), dtype=torch.float16, device=dev)
        v = None if args.variant < 0 else args.variant
        for j in range(args.launches):
            sdt.gemv_f16_m1_kn(x, Ws[j % len(Ws)], y, variant=v)
    elif name == "gemvknws":
        x = torch.from_numpy(inputs.decode_activations()).to(dev)
        Ws = [torch.from_numpy(inputs.decode_weights_kn(r)).to(dev)
              for r in range(inputs.DECODE_BUFFERS)]
        y = torch.empty((inputs.DECODE_N,), dtype=torch.float16, device=dev)
        ws = sdt.Workspace(sdt.gemv_kn_workspace_size(inputs.DECODE_N, inputs.DECODE_K),
                           device=dev)
        for j in range(args.launches):
            sdt.gemv_f16_m1_kn_ws(x, Ws[j % len(Ws)], y, workspace=ws)
    elif name.startswith("copy"):
        mb = int(name[4:])
        src = torch.ones((mb * 1024 * 1024 // 2,), dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.launches):
            dst.copy_(src)
    else:
        raise SystemExit(f"unknown --profile kernel {name}")
    torch.cuda.synchronize()
    log(f"profile mode: {args.launches} launches of {name} done")


def main():
    args = parse()
    if args.profile:
        return profile_mode(args)
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: the kernels are measured on a single MI355X "
                                   "(a sharded run would split N across GPUs with no exchange); "
                                   "run with --gpus 1", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from shape_driven_tile_amd import binding as sdt
    from shape_driven_tile_amd import inputs

    sdt.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} CUs={props.multi_processor_count}")

    def dev_tensor(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- inputs, resident in HBM --------------------------------------------
    host = {}
    ops = {}
    for n in SIZES:
        A, B = inputs.square_operands(n, SEED_INDEX[n])
        host[n] = (A, B)
        ops[n] = (dev_tensor(A), dev_tensor(B), torch.empty((n, n), dtype=torch.float16, device=dev))
    x_h = inputs.decode_activations()
    W_h = [inputs.decode_weights(r) for r in range(inputs.DECODE_BUFFERS)]
    x = dev_tensor(x_h)
    Ws = [dev_tensor(w) for w in W_h]
    y = torch.empty((inputs.DECODE_N,), dtype=torch.float16, device=dev)
    x2 = x.view(1, -1)
    y2 = y.view(1, -1)
    log("inputs resident")

    flop_gemm = {n: 2.0 * n ** 3 for n in SIZES}
    K_dec, N_dec = inputs.DECODE_K, inputs.DECODE_N
    flop_gemv = 2.0 * K_dec * N_dec
    bytes_gemv = 2.0 * K_dec * N_dec           # weight bytes per launch (the pages' GB/s)
    bytes_gemv_all = 2.0 * (K_dec * N_dec + K_dec + N_dec)
    flop_step = sum(flop_gemm.values()) + flop_gemv

    # mark(k): record event k of the step; 0 and 1 bracket the 8192^3 launch,
    # 1 and 2 the decode GEMV (which follows it directly)
    def step(i, mark=None):
        for n in SIZES:
            A, B, C = ops[n]
            if mark is not None and n == DOMINANT:
                mark(0)
                sdt.gemm_f16(A, B, C)
                mark(1)
            else:
                sdt.gemm_f16(A, B, C)
        sdt.gemm_f16(x2, Ws[i % inputs.DECODE_BUFFERS], y2)   # M=1 -> streaming GEMV
        if mark is not None:
            mark(2)

    # ---- parity gate ----------------------------------------------------------
    # C starts NaN-filled, so an element the kernels never write cannot pass.
    # Every element of every square product up to 4096^3 is compared with the
    # oracle; at 8192^3 the whole rows the CPU baseline computes (or 512
    # seeded rows with --no-cpu-baseline).
    import oracle
    for n in SIZES:
        ops[n][2].fill_(float("nan"))
    y.fill_(float("nan"))
    step(0)
    torch.cuda.synchronize()
    gate = {}
    for n in SIZES:
        if n == DOMINANT:
            continue
        A, B = host[n]
        gate[f"gemm_{n}_full"] = outside_tolerance(ops[n][2].cpu().numpy(), oracle.gemm(A, B))
    A, B = host[DOMINANT]
    if args.no_cpu_baseline:
        base, rows, ref = None, gate_rows(DOMINANT, 512), None
        ref = oracle.gemm(np.ascontiguousarray(A[rows]), B)
    else:
        base, rows, ref = cpu_baseline(oracle, host[DOMINANT], args.cpu_seconds)
    gate[f"gemm_{DOMINANT}_rows"] = outside_tolerance(ops[DOMINANT][2].cpu().numpy()[rows], ref)
    gate[f"gemm_{DOMINANT}_rows_checked"] = len(rows)
    del ref
    bad_dec = 0
    for r in range(inputs.DECODE_BUFFERS):
        y.fill_(float("nan"))
        sdt.gemm_f16(x2, Ws[r], y2)
        torch.cuda.synchronize()
        bad_dec += outside_tolerance(y.cpu().numpy(), oracle.gemv_m1(x_h, W_h[r]))
    gate["gemv_8_buffers"] = bad_dec
    failed = gate_failure(gate)
    if failed:
        print(json.dumps(failed), flush=True)
        sys.exit(1)
    log(f"parity gate passed: {gate}")

    # ---- warm-up and the timed region ---------------------------------------
    t0 = time.time()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    warmup_s = time.time() - t0
    log(f"warm-up {args.warmup} steps in {warmup_s:.2f} s")

    evs = StepEvents(torch, args.steps, 3)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i, evs.marker(i))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    dom_ms = [evs.elapsed_ms(i, 0, 1) for i in range(args.steps)]
    dec_ms = [evs.elapsed_ms(i, 1, 2) for i in range(args.steps)]
    evs.close()
    dom_avg_us = 1e3 * sum(dom_ms) / len(dom_ms)
    dec_avg_us = 1e3 * sum(dec_ms) / len(dec_ms)
    value = flop_step / (ms_per_step * 1e-3) / 1e12
    achieved = flop_gemm[DOMINANT] / (dom_avg_us * 1e-6) / 1e12
    log(f"step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s; {DOMINANT}^3 {dom_avg_us:.1f} us "
        f"= {achieved:.1f} TFLOP/s; decode {dec_avg_us:.2f} us")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_s": round(warmup_s, 2),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded uniform[-1,1] fp16 operands; N(0,0.02) fp16 decode weights)",
        "config": {
            "workload": ("square fp16 GEMM C=A.B (A row-major, B K-major, fp32 accumulate, "
                         "fp16 out) at M=N=K in {256,512,768,1024,1536,2048,4096,8192}, then "
                         "M=1 decode GEMV K=4096 N=12288 over 8 rotating weight buffers"),
            "flop_per_step": flop_step,
            "device": props.name or None,
            "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count,
            "tiles": {str(n): sdt.pick_tile(n, n, n, props.multi_processor_count)["id"]
                      for n in SIZES},
        },
        "receipt": receipt(torch),
        "roofline": {
            "bound": "mfma",
            "kernel": f"gemm_pp_kernel (256x256 ping-pong) at {DOMINANT}^3",
            "achieved": round(achieved, 1),
            "peak": round(PEAK_FP16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP16_TFLOPS, 4),
            "traffic": counted_traffic("gemm_pp_256x256_8192_counters.md",
                                       "shape_driven_tile_amd/csrc/gemm_kernel.hpp"),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
            "avg_launch_us": round(dom_avg_us, 2),
            "time_source": (f"{evs.kind} recorded on the launch stream around each {DOMINANT}^3 "
                            "launch of the timed region, averaged over its steps"),
        },
        "decode": {
            "avg_launch_us_in_step": round(dec_avg_us, 3),
            "GBps_in_step": round(bytes_gemv / (dec_avg_us * 1e-6) / 1e9, 1),
            "hbm_frac_in_step": round(bytes_gemv / (dec_avg_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        },
        "gate": {"result": "pass",
                 "checked": (f"every element of C at {', '.join(str(n) for n in SIZES if n != DOMINANT)}"
                             f"^3 (C NaN-filled first); {gate[f'gemm_{DOMINANT}_rows_checked']} "
                             f"whole rows of the {DOMINANT}^3 product; every element of the 8 "
                             "decode products")},
    }

    if not args.no_detail:
        result["detail"] = detail(sdt, torch, np, inputs, ops, x, Ws, y, dev, dev_tensor,
                                  flop_gemm, bytes_gemv, bytes_gemv_all)
        clk = result["detail"].get("clock_under_load") or {}
        if clk.get("mfma_ceiling_at_clock_tflops"):
            # the timed region's 8192^3 rate against 256 CU x 4096 FLOP/clk at
            # the clock sampled in the separate under-load window
            clk["timed_region_frac_of_clock_ceiling"] = round(
                achieved / clk["mfma_ceiling_at_clock_tflops"], 4)
        ceil = (result["detail"].get("mfma_ceiling") or {}).get("uniform") or {}
        if ceil.get("tflops_median"):
            # the timed region's 8192^3 rate against the register-only MFMA
            # loop on operands of the same distribution (no memory traffic)
            result["roofline"]["frac_of_register_only_mfma_rate"] = round(
                achieved / ceil["tflops_median"], 4)
        cold = result["detail"].get("decode_cold") or {}
        if cold.get("us"):
            # the same GEMV alone: graph-replayed over the rotating buffers
            # (no dispatch gap or event in the span), from detail.decode_cold
            result["decode"]["cold_graph_us_median"] = cold["us"]["median"]
            result["decode"]["cold_graph_hbm_frac_median"] = cold.get("hbm_frac_median")

    if base is not None:
        result["cpu_baseline"] = base

    print(json.dumps(result), flush=True)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventCreateWithFlags flag (hip_runtime_api.h)


class StepEvents:
    """Timing events for the launches inside the timed region: `per_step` HIP
    events for each of `steps` steps, recorded on torch's current stream.

    They are created with hipEventDisableSystemFence through the HIP runtime
    torch itself loaded, so recording one takes no system-scope release: a
    default event (torch's) writes back and invalidates the caches when it is
    recorded, which slows the launch after it.  Measured on MI355X with the
    step above: 979 us per step with four torch events, 972 with these, 965
    with none; the decode launch after the 8192^3 one 18.8 us between torch
    events, 17.2 between these.  The stream is synchronized before any
    elapsed time is read.  Where that runtime cannot be found, torch events
    stand in (`kind` says which)."""

    def __init__(self, torch, steps, per_step):
        import ctypes
        self._ct = ctypes
        self._torch = torch
        self._hip = None
        path = None
        try:
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
        except OSError:
            path = None
        if path:
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                    ctypes.c_uint]
            hip.hipEventCreateWithFlags.restype = ctypes.c_int
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventRecord.restype = ctypes.c_int
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.restype = ctypes.c_int
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            hip.hipEventDestroy.restype = ctypes.c_int
            self._hip = hip
            self.kind = "HIP events (hipEventDisableSystemFence)"
            self._ev = []
            for _ in range(steps):
                row = []
                for _ in range(per_step):
                    e = ctypes.c_void_p()
                    rc = hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                     HIP_EVENT_DISABLE_SYSTEM_FENCE)
                    if rc != 0:
                        raise RuntimeError(f"hipEventCreateWithFlags returned {rc}")
                    row.append(e)
                self._ev.append(row)
            self._stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        else:
            self.kind = "torch HIP events"
            self._ev = [[torch.cuda.Event(enable_timing=True) for _ in range(per_step)]
                        for _ in range(steps)]

    def marker(self, i):
        row = self._ev[i]
        if self._hip is None:
            return lambda k: row[k].record()
        hip, stream = self._hip, self._stream

        def mark(k):
            rc = hip.hipEventRecord(row[k], stream)
            if rc != 0:
                raise RuntimeError(f"hipEventRecord returned {rc}")
        return mark

    def elapsed_ms(self, i, a, b) -> float:
        row = self._ev[i]
        if self._hip is None:
            return row[a].elapsed_time(row[b])
        ms = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(ms), row[a], row[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime returned {rc}")
        return ms.value

    def close(self):
        if self._hip is not None:
            for row in self._ev:
                for e in row:
                    self._hip.hipEventDestroy(e)
        self._ev = []


def receipt(torch) -> dict:
    """What the run was made with: the build record written beside libsdt.so
    (git commit, uncommitted changes, compiler), the ROCm release, torch and
    its HIP runtime, the host CPU and this script's own hash."""
    import hashlib
    import platform
    info = {}
    try:
        with open(os.path.join(ROOT, "shape_driven_tile_amd", "build_info.json")) as f:
            info["build"] = json.load(f)
    except (OSError, ValueError):
        info["build"] = None
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    info["torch"] = torch.__version__
    info["hip_runtime"] = getattr(torch.version, "hip", None)
    info["host"] = platform.processor() or platform.machine()
    info["bench_py_sha256_16"] = hashlib.sha256(open(__file__, "rb").read()).hexdigest()[:16]
    return info


def outside_tolerance(got, ref, dtype: str = "f16") -> int:
    """Elements of `got` (values) outside the oracle's acceptance bound around
    `ref` (fp16 output: 1e-2 + 2e-3 |ref|; bf16: the wider bf16 bound); a NaN
    or inf where `ref` is finite counts as outside."""
    import numpy as np
    import oracle
    got = np.asarray(got, dtype=np.float64)
    return int((~(np.abs(got - ref) <= oracle.tolerance(ref, dtype))).sum())


def gate_failure(gate: dict):
    """The JSON record a failed parity gate prints in place of any
    measurement (no value, no throughput), or None when every count of
    elements outside the tolerance is zero."""
    if any(v for k, v in gate.items() if not k.endswith("_checked")):
        return {"metric": METRIC, "value": None, "error": "parity gate failed", "gate": gate}
    return None


def code_sha16(path: str) -> str:
    """sha256[:16] of a C/C++ source with its comments removed and whitespace
    runs collapsed: it changes when the code does, not when a comment does."""
    import hashlib
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def counted_traffic(profile: str, source: str):
    """HBM bytes per launch from a committed counter summary under profiles/
    (FETCH_SIZE + WRITE_SIZE, copy-scaled), or None when the kernel code has
    changed since the counters were taken."""
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
        code = code_sha16(os.path.join(ROOT, source))
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("kernel_code_sha256_16: ", "traffic_bytes_per_launch: ")))
    if fields.get("kernel_code_sha256_16") != code:
        return None
    return float(fields["traffic_bytes_per_launch"])


def _ranges(vals):
    s = sorted(vals)
    return {"min": round(s[0], 3), "median": round(s[len(s) // 2], 3), "max": round(s[-1], 3)}


def time_launches(torch, fn, launches, repeats=10):
    """Per-launch microseconds of `launches` back-to-back calls, `repeats` times."""
    out = []
    for _ in range(repeats):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for j in range(launches):
            fn(j)
        b.record()
        b.synchronize()
        out.append(1e3 * a.elapsed_time(b) / launches)
    return out


PROTOCOL_COLD = ("8 rotating weight buffers (805 MB, past the 256 MB Infinity Cache), ~1 s of "
                 "eager launches to warm up; 200 launches captured in a HIP graph and replayed "
                 "10 times back to back (us: no host launch cost); the same 200 launches issued "
                 "eagerly from Python and event-timed (us_events)")


def cold_times(torch, fn, launches=200):
    """Per-launch microseconds of a rotating-buffer launch fn(j): ~1 s of eager
    launches to warm up, then `launches` calls captured in a HIP graph and
    replayed 10 times back to back (no host launch cost: the reported figure),
    and the same calls issued eagerly from this process, event-timed (beside
    it, for the dispatch gaps)."""
    t0 = time.time()
    j = 0
    while time.time() - t0 < 1.0:
        fn(j)
        j += 1
        if j % 200 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    graph, _ = graph_launches(torch, fn, launches)
    eager = time_launches(torch, fn, launches)
    return graph, eager


def graph_launches(torch, fn, chain, repeats=10):
    """Per-launch microseconds of `chain` calls captured in one HIP graph and
    replayed `repeats` times back to back (graph edges serialize the launches;
    no host launch cost), after ~50 ms of replays to settle the clocks."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for j in range(chain):
                fn(j)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    t_end = time.perf_counter() + 0.05
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(repeats)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [1e3 * a.elapsed_time(b) / chain for a, b in ev], g


def smi_sampler(delay_s=1.0, samples=3, gap_s=0.4):
    """Start a child process that waits `delay_s`, then takes `samples` amd-smi
    readings of GFX clocks, socket power and temperatures `gap_s` apart.  It is
    started before the launches it should see are queued: a reading taken by
    the launching process itself comes only after the queue has drained.
    Returns the process, or None where the tool is not available."""
    import shutil
    import subprocess
    if shutil.which("amd-smi") is None:
        return None
    cmd = f"sleep {delay_s}; for i in $(seq {samples}); do amd-smi metric -c -p -t; sleep {gap_s}; done"
    return subprocess.Popen(["bash", "-c", cmd], stdout=subprocess.PIPE,
                            stderr=subprocess.STDOUT, text=True)


def smi_reading(proc):
    """Collect the sampler's readings: per-XCD clocks (MHz) of every sample,
    their mean, socket power (W) per sample and the last temperatures."""
    import re
    import subprocess
    if proc is None:
        return None
    try:
        out, _ = proc.communicate(timeout=60)
    except subprocess.SubprocessError:
        proc.kill()
        return None
    clocks, power, temps = [], [], {}
    for blk in out.split("GPU: ")[1:]:
        c = [int(m) for m in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*(\d+)\s*MHz", blk)]
        if c:
            clocks.append(round(sum(c) / len(c), 1))
        pw = re.search(r"SOCKET_POWER:\s*(\d+)\s*W", blk)
        if pw:
            power.append(int(pw.group(1)))
        temps = {k.lower(): int(v) for k, v in
                 re.findall(r"(EDGE|HOTSPOT|MEM):\s*(\d+)\s*\S*C", blk)} or temps
    if not clocks and not power:
        return None
    return {"gfx_clk_mhz_per_sample": clocks,
            "gfx_clk_mhz_mean": round(sum(clocks) / len(clocks), 1) if clocks else None,
            "socket_power_w_per_sample": power, "temperature_c": temps}


def detail(sdt, torch, np, inputs, ops, x, Ws, y, dev, dev_tensor, flop_gemm, bytes_gemv,
           bytes_gemv_all):
    det = {"square": {}, "square_graph": {}, "k_sweep": {}, "decode_cold": {}}
    # launch floor: an empty kernel, eager and graph-replayed
    e = (lambda j: sdt.empty_kernel())
    for j in range(200):
        e(j)
    eager = time_launches(torch, e, 200)
    graph, _ = graph_launches(torch, e, 200)
    det["launch_floor"] = {"eager_us": _ranges(eager), "graph_us": _ranges(graph),
                           "kernel": "sdt_empty_kernel (1 workgroup, no memory access)"}
    log(f"launch floor: eager {sorted(eager)[5]:.2f} us, graph {sorted(graph)[5]:.2f} us")
    # every square size as a graph of back-to-back launches; one more replay
    # into a cleared C must reproduce the eager result bit for bit
    for n, (A, B, C) in ops.items():
        chain = 200 if n <= 2048 else (20 if n == 4096 else 5)
        sdt.gemm_f16(A, B, C)
        torch.cuda.synchronize()
        ref = C.clone()
        us, g = graph_launches(torch, (lambda j, A=A, B=B, C=C: sdt.gemm_f16(A, B, C)), chain)
        C.zero_()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(C.view(torch.int16), ref.view(torch.int16)))
        med = sorted(us)[len(us) // 2]
        det["square_graph"][str(n)] = {
            "us": _ranges(us), "launches_per_graph": chain,
            "tflops_median": round(flop_gemm[n] / (med * 1e-6) / 1e12, 1),
            "peak_frac_median": round(flop_gemm[n] / (med * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4),
            "replay_matches_eager": same,
        }
        log(f"square {n} (graph): median {med:.2f} us {det['square_graph'][str(n)]['tflops_median']}"
            f" TFLOP/s{'' if same else '  REPLAY MISMATCH'}")
    # clocks and power while the dominant product runs: ~3.5 s of launches
    # queued, sampled from 1 s in by a process started before the queue
    A, B, C = ops[DOMINANT]
    sampler = smi_sampler()
    for _ in range(5000):
        sdt.gemm_f16(A, B, C)
    torch.cuda.synchronize()
    smi = smi_reading(sampler)
    if smi:
        det["clock_under_load"] = smi
        if smi.get("gfx_clk_mhz_mean"):
            ceil = 256 * 4096 * smi["gfx_clk_mhz_mean"] * 1e6 / 1e12
            det["clock_under_load"]["mfma_ceiling_at_clock_tflops"] = round(ceil, 1)
        log(f"under load: {smi}")
    det["mfma_ceiling"] = mfma_ceiling(sdt, torch, np, inputs, dev_tensor,
                                       props_cus(torch, dev))
    for n, (A, B, C) in ops.items():
        launches = 200 if n <= 2048 else (50 if n == 4096 else 20)
        f = (lambda j, A=A, B=B, C=C: sdt.gemm_f16(A, B, C))
        for j in range(max(20, launches)):
            f(j)
        us = time_launches(torch, f, launches)
        med = sorted(us)[len(us) // 2]
        det["square"][str(n)] = {
            "us": _ranges(us),
            "tflops_median": round(flop_gemm[n] / (med * 1e-6) / 1e12, 1),
            "peak_frac_median": round(flop_gemm[n] / (med * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4),
            "tile": sdt.pick_tile(n, n, n, 0)["id"],
        }
        log(f"square {n}: median {med:.2f} us {det['square'][str(n)]['tflops_median']} TFLOP/s")
    # K sweep at M=N=2048: the default arm at every K, plus both stagger arms
    # forced at K=2048, the one K whose k-tile count allows a stagger; every
    # arm graph-replayed (200 launches per graph, 10 replays), as the squares
    # above, so host launch cost does not blur the per-K differences.
    for K in inputs.K_SWEEP_K:
        A, B = inputs.square_operands(inputs.K_SWEEP_MN, 3, k=K)
        dA, dB = dev_tensor(A), dev_tensor(B)
        C = torch.empty((2048, 2048), dtype=torch.float16, device=dev)
        arms = {"auto": (-1, -1)}
        if sdt.stagger_eligible(K):
            arms["stagger_off"] = (-1, 0)
            arms["stagger_on"] = (-1, 1)
        for name, (tile, st) in arms.items():
            f = (lambda j, tile=tile, st=st: sdt.gemm_f16_ex(dA, dB, C, tile_id=tile, stagger=st))
            us, _ = graph_launches(torch, f, 200)
            med = sorted(us)[len(us) // 2]
            det["k_sweep"][f"{K}_{name}"] = {
                "us": _ranges(us), "timing": "graph replay, 200 launches x 10",
                "tflops_median": round(2.0 * 2048 * 2048 * K / (med * 1e-6) / 1e12, 1),
                "stagger": bool(st == 1 or (st == -1 and sdt.pick_tile(2048, 2048, K, 0)["stagger"])),
                "tile": sdt.pick_tile(2048, 2048, K, 0)["id"],
            }
            log(f"K sweep {K} {name}: median {med:.2f} us")
    # Cold-cache decode: 8 rotating 100.7 MB weight buffers (805 MB >> 256 MB
    # Infinity Cache), ~1 s warm-up, 200 launches x 10 repeats.
    x2, y2 = x.view(1, -1), y.view(1, -1)
    g = (lambda j: sdt.gemm_f16(x2, Ws[j % len(Ws)], y2))
    us, us_ev = cold_times(torch, g)
    med = sorted(us)[len(us) // 2]
    det["decode_cold"] = {
        "us": _ranges(us),
        "us_events": _ranges(us_ev),
        "GBps_weights_median": round(bytes_gemv / (med * 1e-6) / 1e9, 1),
        "GBps_all_median": round(bytes_gemv_all / (med * 1e-6) / 1e9, 1),
        "hbm_frac_median": round(bytes_gemv / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "protocol": PROTOCOL_COLD,
    }
    log(f"decode cold: median {med:.2f} us = {det['decode_cold']['GBps_weights_median']} GB/s")
    # The streaming-read ceiling for the same rotation: the library's read-only
    # kernel (the GEMV's load pattern and nothing else), same protocol.
    words = torch.empty(int(bytes_gemv) // 8192, dtype=torch.int32, device=dev)
    r = (lambda j: sdt.stream_read(Ws[j % len(Ws)], words))
    us_r, us_r_ev = cold_times(torch, r)
    med_r = sorted(us_r)[len(us_r) // 2]
    det["decode_read_ceiling"] = {
        "us": _ranges(us_r),
        "us_events": _ranges(us_r_ev),
        "GBps_median": round(bytes_gemv / (med_r * 1e-6) / 1e9, 1),
        "hbm_frac_median": round(bytes_gemv / (med_r * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "gemv_frac_of_ceiling_median": round(med_r / med, 4),
        "kernel": "sdt_stream_read: 8 KB per wave, 8 non-temporal 16-byte loads per lane, "
                  "no arithmetic or output beyond one word per 8 KB",
        "protocol": PROTOCOL_COLD,
    }
    log(f"decode read ceiling: median {med_r:.2f} us = "
        f"{det['decode_read_ceiling']['GBps_median']} GB/s; the GEMV reaches "
        f"{100 * med_r / med:.1f}% of it")
    # An independent streaming-read reference: a grid-stride read (a plain
    # bandwidth-test pattern, not either GEMV's) over the same rotation, with
    # 32 workgroups of 256 threads per CU.
    nwg = 32 * props_cus(torch, dev)
    words_g = torch.empty(nwg, dtype=torch.int32, device=dev)
    rg = (lambda j: sdt.stream_read_grid(Ws[j % len(Ws)], words_g, nwg))
    us_g, us_g_ev = cold_times(torch, rg)
    med_g = sorted(us_g)[len(us_g) // 2]
    det["decode_read_ceiling_grid"] = {
        "us": _ranges(us_g),
        "us_events": _ranges(us_g_ev),
        "GBps_median": round(bytes_gemv / (med_g * 1e-6) / 1e9, 1),
        "hbm_frac_median": round(bytes_gemv / (med_g * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "gemv_frac_of_ceiling_median": round(med_g / med, 4),
        "kernel": f"sdt_stream_read_grid: {nwg} workgroups of 256 threads, grid-stride, four "
                  "non-temporal 16-byte loads per lane per pass",
        "protocol": PROTOCOL_COLD,
    }
    log(f"decode grid-stride read ceiling: median {med_g:.2f} us = "
        f"{det['decode_read_ceiling_grid']['GBps_median']} GB/s; the GEMV reaches "
        f"{100 * med_g / med:.1f}% of it")

    # The same decode product with the weights stored as K rows of N (the
    # pages' B-layout): gated against the oracle, then the same cold protocol
    # for every instantiation (variant 0 is the default).
    import oracle
    x_h = inputs.decode_activations()
    Wkn_h = [inputs.decode_weights_kn(r) for r in range(inputs.DECODE_BUFFERS)]
    Wkn = [dev_tensor(w) for w in Wkn_h]
    det["decode_kn_cold"] = {"variants": {}}
    for v in range(sdt.gemv_kn_num_variants()):
        bad = 0
        for r in range(inputs.DECODE_BUFFERS):
            sdt.gemv_f16_m1_kn(x, Wkn[r], y, variant=v)
            torch.cuda.synchronize()
            bad += outside_tolerance(y.cpu().numpy(), oracle.gemv_kn(x_h, Wkn_h[r]))
        if bad:
            det["decode_kn_cold"]["variants"][str(v)] = {"gate": f"{bad} outside tolerance"}
            log(f"decode [K][N] variant {v}: PARITY FAILED ({bad}), not timed")
            continue
        h = (lambda j, v=v: sdt.gemv_f16_m1_kn(x, Wkn[j % len(Wkn)], y, variant=v))
        us, us_ev = cold_times(torch, h)
        med = sorted(us)[len(us) // 2]
        det["decode_kn_cold"]["variants"][str(v)] = {
            "us": _ranges(us),
            "us_events": _ranges(us_ev),
            "GBps_weights_median": round(bytes_gemv / (med * 1e-6) / 1e9, 1),
            "hbm_frac_median": round(bytes_gemv / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "gate": "pass",
        }
        log(f"decode [K][N] variant {v}: median {med:.2f} us = "
            f"{det['decode_kn_cold']['variants'][str(v)]['GBps_weights_median']} GB/s")
    # the same product split over K through a workspace (gemv_f16_m1_kn_ws)
    ws_kn = sdt.Workspace(sdt.gemv_kn_workspace_size(inputs.DECODE_N, inputs.DECODE_K), device=dev)
    bad = 0
    for r in range(inputs.DECODE_BUFFERS):
        sdt.gemv_f16_m1_kn_ws(x, Wkn[r], y, workspace=ws_kn)
        torch.cuda.synchronize()
        bad += outside_tolerance(y.cpu().numpy(), oracle.gemv_kn(x_h, Wkn_h[r]))
    if bad:
        det["decode_kn_cold"]["split_ws"] = {"gate": f"{bad} outside tolerance"}
        log(f"decode [K][N] split over K: PARITY FAILED ({bad}), not timed")
    else:
        h = (lambda j: sdt.gemv_f16_m1_kn_ws(x, Wkn[j % len(Wkn)], y, workspace=ws_kn))
        us, us_ev = cold_times(torch, h)
        med = sorted(us)[len(us) // 2]
        det["decode_kn_cold"]["split_ws"] = {
            "us": _ranges(us),
            "us_events": _ranges(us_ev),
            "GBps_weights_median": round(bytes_gemv / (med * 1e-6) / 1e9, 1),
            "hbm_frac_median": round(bytes_gemv / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "workspace_bytes": ws_kn.nbytes,
            "gate": "pass (all 8 buffers)",
            "what": "gemv_f16_m1_kn_ws: 256-column bands, K split so ~768 workgroups stream, "
                    "then a second kernel adds the splits in order (both kernels timed)",
        }
        log(f"decode [K][N] split over K: median {med:.2f} us = "
            f"{det['decode_kn_cold']['split_ws']['GBps_weights_median']} GB/s")
    # read ceilings of the [K][N] access pattern: the same 8 weight buffers read
    # in runs of 128 bytes per row (the one-launch kernel's bands) and 512 bytes
    # (the split kernel's), with one workgroup per band or K cut into chunks
    row_bytes = inputs.DECODE_N * 2
    runs = {}
    out_w = torch.empty((1 << 16,), dtype=torch.int32, device=dev)
    for run, rpw in ((128, inputs.DECODE_K), (128, 256), (512, 256), (512, 64)):
        h = (lambda j, run=run, rpw=rpw: sdt.stream_read_runs(
            Wkn[j % len(Wkn)], inputs.DECODE_K, row_bytes, run, rpw, out_w))
        us, us_ev = cold_times(torch, h)
        med = sorted(us)[len(us) // 2]
        runs[f"{run}B_rows_per_wg_{rpw}"] = {
            "workgroups": (row_bytes // run) * (inputs.DECODE_K // rpw),
            "us": _ranges(us),
            "us_events": _ranges(us_ev),
            "GBps_median": round(bytes_gemv / (med * 1e-6) / 1e9, 1),
        }
        log(f"[K][N] read in {run}-byte runs, {rpw} rows per workgroup: median {med:.2f} us = "
            f"{runs[f'{run}B_rows_per_wg_{rpw}']['GBps_median']} GB/s")
    det["decode_kn_cold"]["read_runs"] = runs
    det["decode_kn_cold"]["protocol"] = "weights as K rows of N; " + PROTOCOL_COLD
    det["bf16"] = detail_bf16(sdt, torch, np, inputs, oracle, dev, flop_gemm, bytes_gemv)
    det["ksplit"] = detail_ksplit(sdt, torch, np, inputs, oracle, dev)
    return det


MFMA_CEILING_ITERS = 1000   # ~1.2 ms per launch on 256 CUs at the power limit


def mfma_ceiling(sdt, torch, np, inputs, dev_tensor, cus):
    """The matrix cores' own rate on the GEMM's operand distribution: the
    library's register-only MFMA loop (the 256 x 256 kernel's MFMA phase, 8
    waves per CU, no memory traffic) on uniform [-1,1] fp16 fragments with the
    kernel's v_mfma_f32_16x16x32_f16, the same with v_mfma_f32_32x32x16_f16,
    on all-ones fragments, and on uniform bf16 ones; each after ~2 s of
    launches (the power limit's steady state), then 20 launches per graph
    replayed 5 times; clocks sampled while the first runs."""
    flop = float(cus) * MFMA_CEILING_ITERS * sdt.MFMA_CEILING_FLOP_PER_ITER
    out = torch.empty((cus * 512,), dtype=torch.float32, device="cuda:0")
    res = {"kernel": "sdt_mfma_ceiling: 8 waves per workgroup, 2^20 FLOP per wave per "
                     "iteration (64 v_mfma_f32_16x16x32 or 32 v_mfma_f32_32x32x16 on the 24 "
                     "fragments of one k-tile of the 256x256 kernel's wave, no memory access), "
                     f"{cus} workgroups, {MFMA_CEILING_ITERS} iterations",
           "flop_per_launch": flop}
    n = 24 * 64 * 8
    arms = (("uniform", inputs.uniform_f16((n,), 5000), False, False),
            ("uniform_32x32x16", inputs.uniform_f16((n,), 5000), False, True),
            ("ones", np.ones((n,), dtype=np.float16), False, False),
            ("uniform_bf16", inputs.uniform_bf16((n,), 5000), True, False))
    for name, frags_h, bf16, mfma32 in arms:
        frags = dev_tensor(frags_h.view(np.uint16))
        f = (lambda j, frags=frags, bf16=bf16, mfma32=mfma32:
             sdt.mfma_ceiling(frags, MFMA_CEILING_ITERS, out, cus, bf16=bf16, mfma32=mfma32))
        sampler = smi_sampler() if name == "uniform" else None
        t0 = time.time()
        while time.time() - t0 < 2.0:
            for _ in range(100):
                f(0)
            torch.cuda.synchronize()
        us, _ = graph_launches(torch, f, 20, repeats=5)
        med = sorted(us)[len(us) // 2]
        res[name] = {"us": _ranges(us),
                     "tflops_median": round(flop / (med * 1e-6) / 1e12, 1),
                     "peak_frac_median": round(flop / (med * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4)}
        if sampler is not None:
            smi = smi_reading(sampler)
            if smi:
                res[name]["clock_under_load"] = smi
        log(f"mfma ceiling ({name}): median {med:.1f} us {res[name]['tflops_median']} TFLOP/s")
    return res


def props_cus(torch, dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


# shapes of the k-split detail: long k-loops over few output tiles, where the
# workspace entry point splits K, and two of the benchmarked squares, where
# it does not (its plan is gemm_f16's)
KSPLIT_SHAPES = ((256, 256, 16384), (128, 128, 65536), (512, 512, 8192), (384, 384, 12288),
                 (1024, 1024, 1024), (1536, 1536, 1536))


def detail_ksplit(sdt, torch, np, inputs, oracle, dev):
    """gemm_f16 against gemm_f16_ws (k-split across workgroups where its plan
    takes one) on the same inputs: every element gated against the oracle,
    then both graph-timed."""
    out = {}
    for (M, N, K) in KSPLIT_SHAPES:
        A = inputs.uniform_f16((M, K), 61)
        B = inputs.uniform_f16((N, K), 62)
        dA = torch.from_numpy(A).to(dev)
        dB = torch.from_numpy(B).to(dev)
        C = torch.empty((M, N), dtype=torch.float16, device=dev)
        need = sdt.gemm_workspace_size(M, N, K)
        ws = sdt.Workspace(max(need, 16), device=dev)
        plan = sdt.pick_tile_ws(M, N, K, 0, ws.nbytes)
        C.fill_(float("nan"))
        sdt.gemm_f16_ws(dA, dB, C, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.gemm(A, B)
        bad = outside_tolerance(C.cpu().numpy(), ref)
        key = f"{M}x{N}x{K}"
        if bad:
            out[key] = {"gate": f"{bad} outside tolerance"}
            log(f"k-split {key}: PARITY FAILED ({bad}), not timed")
            continue
        flop = 2.0 * M * N * K
        chain = max(4, min(200, int(2e12 / flop)))
        us_p, _ = graph_launches(torch, (lambda j: sdt.gemm_f16(dA, dB, C)), chain)
        us_w, _ = graph_launches(torch, (lambda j: sdt.gemm_f16_ws(dA, dB, C, workspace=ws)), chain)
        mp, mw = sorted(us_p)[len(us_p) // 2], sorted(us_w)[len(us_w) // 2]
        out[key] = {"gate": "pass (every element)", "gemm_f16_us": _ranges(us_p),
                    "gemm_f16_ws_us": _ranges(us_w),
                    "plan_ws": {k: plan[k] for k in ("id", "splits", "split_algo", "stages",
                                                     "kgroups")},
                    "workspace_bytes": need, "speedup_median": round(mp / mw, 3),
                    "timing": f"graph replay, {chain} launches x 10"}
        log(f"k-split {key}: gemm_f16 {mp:.2f} us, gemm_f16_ws {mw:.2f} us "
            f"(splits {plan['splits']})")
        del dA, dB, C, ws
    return out


def detail_bf16(sdt, torch, np, inputs, oracle, dev, flop_gemm, bytes_gemv):
    """The bfloat16 entry points on the same shapes: a sampled oracle gate,
    then graph-timed squares and the cold decode protocol."""
    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    out = {"square_graph": {}, "decode_cold": {}}
    for n in SIZES:
        A, B = inputs.square_operands_bf16(n, SEED_INDEX[n])
        dA, dB = to_dev(A), to_dev(B)
        C = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
        sdt.gemm_bf16(dA, dB, C)
        torch.cuda.synchronize()
        rng = np.random.default_rng(n + 1)
        r = rng.integers(0, n, 1024)
        c = rng.integers(0, n, 1024)
        ref = oracle.gemm_sample(A, B, r, c, dtype="bf16")
        bad = outside_tolerance(oracle.bf16_decode(bits(C)[r, c]), ref, "bf16")
        if bad:
            out["square_graph"][str(n)] = {"gate": f"{bad} of 1024 sampled outside tolerance"}
            log(f"bf16 square {n}: PARITY FAILED ({bad}), not timed")
            continue
        chain = 200 if n <= 2048 else (20 if n == 4096 else 5)
        us, _ = graph_launches(torch, (lambda j, dA=dA, dB=dB, C=C: sdt.gemm_bf16(dA, dB, C)), chain)
        med = sorted(us)[len(us) // 2]
        out["square_graph"][str(n)] = {
            "us": _ranges(us), "launches_per_graph": chain, "gate": "pass",
            "tflops_median": round(flop_gemm[n] / (med * 1e-6) / 1e12, 1),
            "peak_frac_median": round(flop_gemm[n] / (med * 1e-6) / 1e12 / PEAK_FP16_TFLOPS, 4),
        }
        log(f"bf16 square {n} (graph): median {med:.2f} us "
            f"{out['square_graph'][str(n)]['tflops_median']} TFLOP/s")
        del dA, dB, C
    x_h = inputs.decode_activations_bf16()
    W_h = [inputs.decode_weights_bf16(r) for r in range(inputs.DECODE_BUFFERS)]
    x = to_dev(x_h)
    Ws = [to_dev(w) for w in W_h]
    y = torch.empty((inputs.DECODE_N,), dtype=torch.bfloat16, device=dev)
    bad = 0
    for r in range(inputs.DECODE_BUFFERS):
        sdt.gemv_bf16_m1(x, Ws[r], y)
        torch.cuda.synchronize()
        ref = oracle.gemv_m1(x_h, W_h[r], dtype="bf16")
        bad += outside_tolerance(oracle.bf16_decode(bits(y)), ref, "bf16")
    if bad:
        out["decode_cold"] = {"gate": f"{bad} outside tolerance"}
        log(f"bf16 decode: PARITY FAILED ({bad}), not timed")
        return out
    g = (lambda j: sdt.gemv_bf16_m1(x, Ws[j % len(Ws)], y))
    us, us_ev = cold_times(torch, g)
    med = sorted(us)[len(us) // 2]
    out["decode_cold"] = {
        "us": _ranges(us), "us_events": _ranges(us_ev), "gate": "pass",
        "GBps_weights_median": round(bytes_gemv / (med * 1e-6) / 1e9, 1),
        "hbm_frac_median": round(bytes_gemv / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
        "protocol": "bf16 weights; " + PROTOCOL_COLD,
    }
    log(f"bf16 decode cold: median {med:.2f} us = {out['decode_cold']['GBps_weights_median']} GB/s")
    return out


def gate_rows(n, count, seed=8192):
    """`count` distinct sorted row indices of an n-row product: the first and
    last row of every 256-row tile band, the rest drawn from a seeded
    generator."""
    import numpy as np
    rng = np.random.default_rng(seed)
    pick = {0, n - 1}
    if count >= 2 * (n // 256):
        for b in range(0, n, 256):
            pick.update((b, b + 255))
    while len(pick) < min(count, n):
        pick.update(int(v) for v in rng.integers(0, n, count - len(pick)))
    return np.array(sorted(pick)[:count], dtype=np.int64)


def cpu_baseline(oracle, AB, target_s):
    """The oracle, untuned, on a bounded sample of the dominant product: whole
    output rows of the 8192^3 GEMM (gate_rows: every tile band's edges plus
    seeded rows), as many as take about target_s seconds.  Returns the
    baseline record, the row indices and the oracle's rows, which the parity
    gate compares with the GPU's."""
    import numpy as np
    A, B = AB
    n = A.shape[0]
    threads = oracle.max_threads()
    # rate estimate on enough rows to occupy every thread
    est = min(n, 8 * threads)
    t = time.time()
    oracle.gemm(np.ascontiguousarray(A[:est]), B)
    per_row = max((time.time() - t) / est, 1e-6)
    rows = int(min(n, max(512, est, target_s / per_row)))
    idx = gate_rows(n, rows)
    a_rows = np.ascontiguousarray(A[idx])
    t = time.time()
    ref = oracle.gemm(a_rows, B)
    dt = time.time() - t
    flop = 2.0 * rows * n * n
    # one thread at two small squares, for scale
    one_thread = {}
    for m in (256, 1024):
        a = np.ascontiguousarray(A[:m, :m])
        b = np.ascontiguousarray(B[:m, :m])
        t = time.time()
        oracle.gemm(a, b, threads=1)
        d1 = time.time() - t
        one_thread[f"{m}^3"] = {"s": round(d1, 4), "GFLOP_s": round(2.0 * m ** 3 / d1 / 1e9, 3)}
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    rec = {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "kind": "oracle",
           "sample": f"{rows} whole output rows of the {n}^3 product ({flop:.3g} FLOP) in "
                     f"{dt:.2f} s, fp64 accumulation, {threads} OpenMP threads; the same rows "
                     "are the parity gate's check of the GPU's {n}^3 result".replace("{n}", str(n)),
           "GFLOP_s": round(flop / dt / 1e9, 3), "cpu_model": model,
           "one_thread": one_thread}
    return rec, idx, ref


if __name__ == "__main__":
    main()
