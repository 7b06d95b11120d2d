#!/usr/bin/env python3
"""Throughput of the weight-only group-quantized matmul on one MI355X.

One step is one decode product y = x @ dequant(W) at M=1, K=4096, N=4096,
4-bit codes, group size 128 (one transformer projection), on seeded synthetic
inputs already resident in HBM, the packed words in the library's load-time
layout (16-column strips: the same words, reordered once by qmm_to_strips so
that each block streams its strip in order; the K-major time of the same
workload is reported beside it). `value` is the achieved HBM bandwidth in GB/s
of the K timed steps: the algorithmic bytes of a step (packed words, scales,
zero points, x and y) over the time per step.

Protocol, the same for every product below:
  * Cold weights: every launch reads a different copy of the packed weights,
    scales and zero points, and the copies together span at least 512 MiB
    (twice the 256 MB Infinity Cache), so each launch streams its weights
    from HBM.
  * Time per step: the timed launches run back to back as kernel nodes of one
    HIP graph, behind a lead-in of the same launch on a copy of its own (about
    300 us, so that they start on a busy GPU at its working clocks). That graph
    and one of the lead-in alone are each replayed after a 640 MiB fill that
    evicts every cache, between events on the launch stream; their difference
    is the time of exactly the timed launches, free of the fixed cost of a
    graph launch (~10 us, which would otherwise weigh on short runs): the
    average launch duration over the timed region, each node's dispatch
    included, no host overhead (a rocprofv3 kernel trace of the same nodes
    reports the same durations, to a few %). Median of three.
    `roofline.achieved` is the algorithmic bytes (or flops) of one launch
    over it.
  * Floors: a plain streaming read of the same byte count, cold, timed the
    same way (best of a few launch shapes), an empty kernel, and a dense
    MFMA loop.

The JSON line holds the headline (`value`, exactly --steps steps after
--warmup untimed ones) and, under `configs`, every workload at a fixed count
of steps independent of --steps (200 per decode product, 40 per prefill
product after 100 untimed launches, past a clock transient of back-to-back
prefill launches):
  configs[*]    per workload (weights K-major, as packed): time per step, GB/s
                and TFLOP/s, the roofline of its kernel (traffic from the
                committed counter summary of that kernel source, else null),
                the streaming-read floor of its bytes, and the launch plan
  strips[*]     the same workloads with the weights in 16-column strips
  gemm_int4_g128  the prefill shape again with 4-bit codes in groups of 128
  bf16          the headline decode and the prefill products with bf16 data
  readme_shapes the prefill kernel at the README's benchmark shapes (4-bit g128)
  floors        an empty kernel as a graph node, a dense MFMA loop
  cpu_baseline  the CPU oracle on the headline workload on this host's cores
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_DENSE_PEAK_TFLOPS = 2500.0  # bf16 is the same
COLD_BYTES = 512 * 1024 * 1024  # twice the Infinity Cache
SCRUB_BYTES = 640 * 1024 * 1024
METRIC = "M=1 GEMV achieved HBM GB/s (% of peak); M=2048 GEMM TOPS (% MFMA peak)"
GEMV_STEPS = 200
LEAD_MAX_NODES, LEAD_US = 64, 300.0  # lead-in before the timed launches
GEMM_STEPS, GEMM_WARMUP = 40, 100
CSRC = os.path.join(ROOT, "weight_only_group_amd", "csrc")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ sizes

def algorithmic_bytes(M, K, N, bits, group_size) -> int:
    """Packed words, scales and zero points once, x once, y once."""
    groups = 1 if group_size == -1 else K // group_size
    return K * N * bits // 8 + 2 * groups * N * 2 + M * K * 2 + M * N * 2


def kernel_sources(kind: str, bits: int) -> list[str]:
    if kind == "gemm":
        return ["gemm.hip", "common.h"]
    return ["gemv.hip", "gemv_common.h", "gemv_wave.h", f"gemv_wave_b{bits}.hip", "common.h"]


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, kind: str, bits: int):
    """HBM bytes per launch from profiles/traffic_<workload>.txt, if taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.loads("".join(line for line in f if not line.startswith("#")))
    except (ValueError, OSError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(kernel_sources(kind, bits)):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ host facts

def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# ------------------------------------------------------------------ timing

class Clock:
    """Average launch duration of back-to-back launches (one graph replay, cold caches)."""

    def __init__(self, torch):
        self.torch = torch
        self.scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda:0")

    def per_step_us(self, launch, steps: int, first: int = 0) -> float:
        """`launch(i, stream)` for i in [first, first + steps), back to back: time per launch.

        The timed launches run in one graph behind a lead-in of the same launch on a copy of
        its own (`launch(-1, stream)`, about LEAD_US long), so that they start on a busy GPU at
        its working clocks. That graph and one of the lead-in alone are each replayed after a
        640 MiB fill that evicts the caches, between events on the launch stream; the
        difference of the two is the time of exactly `steps` launches, free of the fixed cost of
        a graph launch (which would otherwise weigh on short runs). Median of three."""
        torch = self.torch
        sp = torch.cuda.current_stream().cuda_stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        launch(-1, sp)
        e0.record()
        for _ in range(3):
            launch(-1, sp)
        e1.record()
        torch.cuda.synchronize()
        rough = max(e0.elapsed_time(e1) * 1e3 / 3, 0.5)
        nlead = max(2, min(LEAD_MAX_NODES, math.ceil(LEAD_US / rough)))

        def capture(n_timed):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                s_ = torch.cuda.current_stream().cuda_stream
                for _ in range(nlead):
                    launch(-1, s_)
                for i in range(first, first + n_timed):
                    launch(i, s_)
            return g

        full, lead = capture(steps), capture(0)
        full.replay()  # untimed: the first replay of a graph carries one-time work
        lead.replay()
        torch.cuda.synchronize()

        def timed(g):
            self.scrub.zero_()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3

        diffs = sorted((timed(full) - timed(lead)) / steps for _ in range(3))
        del full, lead
        return diffs[1]


# ------------------------------------------------------------------ products

class Product:
    """One product's device inputs, rotated weight copies and launch functions."""

    def __init__(self, w, torch, datagen, M, K, N, bits, gs, seed, zero_range, scale_range, bf16=False,
                 name=None, copies=None, strips=False):
        self.w, self.torch = w, torch
        self.M, self.K, self.N, self.bits, self.gs, self.bf16 = M, K, N, bits, gs, bf16
        self.strips = strips
        self.name = (name or f"m{M}_k{K}_n{N}_int{bits}_g{gs}") + ("_strips" if strips else "")
        dev = torch.device("cuda:0")
        wl = datagen.Workload(self.name, M, K, N, bits, gs, zero_range, scale_range, seed)
        d = datagen.generate(wl)
        self.d = d
        if bf16:
            b = datagen.as_bf16_case(d)
            x, z0, s0 = (torch.from_numpy(b[k].view("int16")).view(torch.bfloat16).to(dev)
                         for k in ("x", "zeros", "scales"))
        else:
            x, z0, s0 = (torch.from_numpy(d[k]).to(dev) for k in ("x", "zeros", "scales"))
        qw0, qlo0 = w.qmm_pack(torch.from_numpy(d["codes"]).to(dev), bits)
        per = qw0.nbytes + z0.nbytes + s0.nbytes + (0 if qlo0 is None else qlo0.nbytes)
        self.R = max(1, math.ceil(COLD_BYTES / per)) if copies is None else copies
        self.copies = [(qw0, qlo0, z0, s0)] + [
            (qw0.clone(), None if qlo0 is None else qlo0.clone(), z0.clone(), s0.clone()) for _ in range(self.R - 1)]
        # a copy of its own for the lead-in launches before a timed replay
        self.lead = (qw0.clone(), None if qlo0 is None else qlo0.clone(), z0.clone(), s0.clone())
        if strips:  # the load-time re-layout of every copy into 16-column strips
            conv = lambda t: None if t is None else w.qmm_to_strips(t)
            self.copies = [(conv(a), conv(b), c, e) for a, b, c, e in self.copies]
            self.lead = (conv(self.lead[0]), conv(self.lead[1]), self.lead[2], self.lead[3])
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        self.x = x
        self.y = torch.empty((M, N), dtype=x.dtype, device=dev)
        self.gemv = M <= 16
        lib = w.library()
        self.lib = lib
        sfx = "_ex" if strips else ("_bf16" if bf16 else "")
        self.flags = ((w.QMM_BF16 if bf16 else 0) | w.QMM_STRIPS) if strips else None
        if self.gemv:
            nb = w.workspace_bytes(M, K, N, bits, gs)
            self.ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev)
            self.fn = getattr(lib, "qmm_gemv" + sfx)
            self.plan = w.gemv_plan_info(M, K, N, bits, gs)
        else:
            self.fn = getattr(lib, "qmm_gemm" + sfx)
            self.plan = w.gemm_plan_info(M, K, N, bits, gs)
        self.bytes = algorithmic_bytes(M, K, N, bits, gs)
        self.flops = 2.0 * M * K * N

    def launch(self, i: int, sp: int):
        qw, qlo, z, s = self.lead if i < 0 else self.copies[i % self.R]
        args = [self.x.data_ptr(), self.M, self.K, qw.data_ptr(), None if qlo is None else qlo.data_ptr(),
                z.data_ptr(), s.data_ptr(), None, self.N, self.bits, self.gs]
        if self.flags is not None:
            args.append(self.flags)
        args.append(self.y.data_ptr())
        if self.gemv:
            args += [self.ws.data_ptr(), self.ws.numel()]
        st = self.fn(*args, sp)
        if st != 0:
            raise RuntimeError(f"{self.name}: {self.lib.qmm_last_error().decode()}")

    def kernel_name(self) -> str:
        p = self.plan
        if self.gemv and p["kernel"] == 1:
            return (f"gemv_wave_kernel<bits={self.bits}, vec={p['vec']}, waves={p['waves']}, units={p['units']}, "
                    f"groups/wave={p['groups_per_wave']}, {'bf16' if self.bf16 else 'f16'}, "
                    f"{'one row' if self.M == 1 else 'rows'}>")
        if self.gemv:
            return f"gemv_kernel<bits={self.bits}, vec={p['vec']}, waves={p['waves']}>, ksplit={p['ksplit']}"
        return f"gemm_kernel<bits={self.bits}, {p['bm']}x{p['bn']} tile, {p['kgroups']} K groups>"

    def free(self):
        self.copies = None
        self.lead = None
        self.torch.cuda.empty_cache()


def measure(clock, prod: Product, steps: int, warmup: int):
    for i in range(max(warmup, 3)):
        prod.launch(i, prod.torch.cuda.current_stream().cuda_stream)
    prod.torch.cuda.synchronize()
    step_us = clock.per_step_us(prod.launch, steps, first=warmup)
    assert bool(prod.torch.isfinite(prod.y).all()), prod.name
    return step_us


def read_floor(torch, clock, probes, nbytes: int, steps: int):
    """A plain cold streaming read of nbytes: average launch duration, best of four launch shapes."""
    nbytes = nbytes // 256 * 256
    R = max(1, math.ceil(COLD_BYTES / nbytes))
    buf = torch.ones(R * nbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")

    def run(blocks, threads):
        def launch(i, sp):
            st = probes.qmm_probe_read(buf.data_ptr() + (i % R) * nbytes, nbytes, blocks, threads, sink.data_ptr(),
                                       sp)
            if st != 0:
                raise RuntimeError(f"probe failed ({st})")
        return launch

    best = None
    for blocks, threads in ((256, 1024), (512, 1024), (1024, 512), (2048, 256)):
        us = clock.per_step_us(run(blocks, threads), steps)
        if best is None or us < best[0]:
            best = (us, blocks, threads)
    us, blocks, threads = best
    del buf
    return {"bytes": nbytes, "us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1), "blocks": blocks,
            "threads": threads}


def probes_library():
    lib = ctypes.CDLL(os.path.join(ROOT, "weight_only_group_amd", "libqmm_probes.so"))
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.qmm_probe_empty.argtypes = [I, I, P]
    lib.qmm_probe_read.argtypes = [P, ctypes.c_size_t, I, I, P, P]
    lib.qmm_probe_mfma.argtypes = [I, I, P, P]
    return lib


def product_entry(prod: Product, steps: int, step_us: float, floor):
    kind = "gemv" if prod.gemv else "gemm"
    e = {
        "workload": prod.name, "path": ("qmm_gemv" if prod.gemv else "qmm_gemm") + ("_ex" if prod.strips else ""),
        "weight_layout": "16-column strips" if prod.strips else "K-major",
        "M": prod.M, "K": prod.K, "N": prod.N, "bits": prod.bits, "group_size": prod.gs,
        "dtype": "bf16" if prod.bf16 else "f16", "steps": steps, "weight_copies_rotated": prod.R,
        "algorithmic_bytes": prod.bytes, "flops": prod.flops,
        "ms_per_step": round(step_us / 1e3, 6), "us_per_launch": round(step_us, 3),
        "GB/s": round(prod.bytes / step_us / 1e3, 1), "TFLOP/s": round(prod.flops / step_us / 1e6, 2),
        "plan": prod.plan,
    }
    traffic = committed_traffic(prod.name, kind, prod.bits) if not prod.bf16 else None
    if prod.gemv:
        ach = prod.bytes / step_us / 1e3
        e["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": prod.kernel_name()}
    else:
        ach = prod.flops / step_us / 1e6
        e["roofline"] = {"bound": "mfma", "achieved": round(ach, 1), "peak": FP16_DENSE_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / FP16_DENSE_PEAK_TFLOPS, 4), "traffic": traffic,
                         "kernel": prod.kernel_name()}
    if floor is not None:
        e["read_floor"] = floor
        e["over_read_floor"] = round(step_us / floor["us"], 3)
    return e


# ------------------------------------------------------------------ extras

README_SHAPES = ((128, 512, 1024, 2.5), (256, 1024, 2048, 8.2), (512, 2048, 4096, 31.5))


def bench_readme_shapes(w, torch, datagen, clock):
    """The prefill kernel at the README's own shapes (M, N, K; 4-bit g128 from its quick start), cold.
    The page quotes A100 latencies for them, context only."""
    out = []
    for M, N, K, page_ms in README_SHAPES:
        p = Product(w, torch, datagen, M, K, N, 4, 128, M + N + K, (0, 15), (0.005, 0.02))
        step_us = measure(clock, p, 200, 3)
        out.append({"M": M, "N": N, "K": K, "bits": 4, "group_size": 128, "us_per_launch": round(step_us, 3),
                    "TFLOP/s": round(p.flops / step_us / 1e6, 2),
                    "tile": f"{p.plan['bm']}x{p.plan['bn']}", "page_context_a100_ms": page_ms})
        p.free()
    return out


def bench_floors(torch, clock, probes):
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda:0")

    def empty(i, sp):
        if probes.qmm_probe_empty(256, 1024, sp) != 0:
            raise RuntimeError("probe failed")

    out = {"empty_kernel_graph_node_us": round(clock.per_step_us(empty, 400), 3)}
    iters, blocks = 4000, 1024
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sp = torch.cuda.current_stream().cuda_stream
    probes.qmm_probe_mfma(blocks, iters, sink.data_ptr(), sp)
    e0.record()
    for _ in range(3):
        probes.qmm_probe_mfma(blocks, iters, sink.data_ptr(), sp)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 3
    flops = blocks * 4 * 4 * iters * 2.0 * 32 * 32 * 16
    out["mfma_32x32x16_f16"] = {"TFLOP/s": round(flops / us / 1e6, 1), "blocks": blocks, "iters": iters}
    return out


def cpu_baseline(datagen, d, wl, seconds: float):
    """The oracle as it stands (unpack, float64 dequantize, product) on the headline workload."""
    import oracle
    qw, qlo = oracle.pack(d["codes"], wl.bits)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.quantized_matmul(d["x"], qw, qlo, d["zeros"], d["scales"], wl.bits, wl.group_size)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": round(algorithmic_bytes(wl.M, wl.K, wl.N, wl.bits, wl.group_size) / per / 1e9, 4),
            "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"the whole headline workload ({wl.name}) from packed words: unpack, float64 dequantize "
                      f"and product; {n} calls in {el:.1f} s, {per * 1e3:.1f} ms each",
            "threads_note": "cores = threads of the BLAS pool the product ran on; unpack and dequantize run on one",
            "os_cpu_count": os.cpu_count(), "cpus_in_affinity": affinity, "cpu_model": cpu_model()}


def cpu_baseline_gemm(datagen, d, wl, rows: int):
    import oracle
    qw, _ = oracle.pack(d["codes"], wl.bits)
    t0 = time.perf_counter()
    oracle.quantized_matmul(d["x"][:rows], qw, None, d["zeros"], d["scales"], wl.bits, wl.group_size)
    el = time.perf_counter() - t0
    return {"value": round(2.0 * rows * wl.N * wl.K / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {wl.M} rows of {wl.name} from packed words (unpack, float64 dequantize of "
                      f"the whole weight, product), one call, {el:.1f} s"}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="timed headline decode products")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget for the baseline")
    ap.add_argument("--cpu-gemm-rows", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the five workloads and the headline")
    ap.add_argument("--only", default=None, metavar="WORKLOAD",
                    help="a few launches of one workload's product, its own short line (for counter profiles)")
    ap.add_argument("--strips", action="store_true", help="with --only: the weights in 16-column strips")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the products, 4 plain device copies of MIB MiB each (outside every timed region), "
                         "so that a counter profile can scale FETCH_SIZE / WRITE_SIZE by a copy of known size")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (no sharding, no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import datagen
    import weight_only_group_amd as w

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w.library()  # fails loudly if the HIP library is missing
    try:
        if args.only:
            run_only(args, torch, datagen, w)
        else:
            run(args, torch, datagen, w)
    finally:
        if args.copy_calibration > 0:
            copy_calibration(torch, args.copy_calibration)


def copy_calibration(torch, mib: int):
    """Four device-to-device copies of `mib` MiB: a reference kernel whose HBM bytes are known exactly."""
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "copies": 4}),
          flush=True)


def workload_product(w, torch, datagen, wl, bf16=False, copies=None, strips=False):
    return Product(w, torch, datagen, wl.M, wl.K, wl.N, wl.bits, wl.group_size, wl.seed, wl.zero_range,
                   wl.scale_range, bf16=bf16, name=wl.name, copies=copies, strips=strips)


def run_only(args, torch, datagen, w):
    """A few cold launches of one workload, for counters that are read per dispatch: one copy of the
    weights, and a 640 MiB fill before each launch evicts it from the caches (few dispatches in all)."""
    wl = datagen.WORKLOADS[args.only]
    p = workload_product(w, torch, datagen, wl, copies=1, strips=args.strips)
    scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda:0")
    sp = torch.cuda.current_stream().cuda_stream
    for i in range(20):
        scrub.zero_()
        p.launch(i, sp)
    torch.cuda.synchronize()
    print(json.dumps({"workload": p.name, "launches": 20, "kernel": p.kernel_name(),
                      "algorithmic_bytes": p.bytes}), flush=True)
    p.free()


def run(args, torch, datagen, w):
    clock = Clock(torch)
    probes = probes_library()
    head_wl = datagen.WORKLOADS[datagen.HEADLINE_GEMV]

    # the headline: exactly --steps steps after --warmup untimed ones, the
    # weights in the decode product's load-time layout (16-column strips)
    head = workload_product(w, torch, datagen, head_wl, strips=True)
    say(f"headline {head.name}: {args.steps} steps after {args.warmup}")
    h_step = measure(clock, head, args.steps, args.warmup)
    head_d = head.d
    head.free()

    configs = []
    gemm_d = None
    for name, wl in datagen.WORKLOADS.items():
        p = workload_product(w, torch, datagen, wl)
        if p.gemv:
            steps, warm = GEMV_STEPS, 20
            step_us = measure(clock, p, steps, warm)
        else:
            steps, warm = GEMM_STEPS, GEMM_WARMUP
            step_us = measure(clock, p, steps, warm)
            gemm_d = p.d
        floor = read_floor(torch, clock, probes, p.bytes, 200 if p.gemv else 20)
        e = product_entry(p, steps, step_us, floor)
        say(f"{name}: {step_us:.3f} us per launch, streaming-read floor {floor['us']:.3f} us, "
            f"frac {e['roofline']['frac']}")
        configs.append(e)
        p.free()

    # the same workloads with their weights re-laid out into 16-column strips
    # at load time (the same words: qmm_gemv_ex / qmm_gemm_ex with QMM_STRIPS)
    strips = []
    for name, wl in datagen.WORKLOADS.items():
        p = workload_product(w, torch, datagen, wl, strips=True)
        steps, warm = (GEMV_STEPS, 20) if p.gemv else (GEMM_STEPS, GEMM_WARMUP)
        step_us = measure(clock, p, steps, warm)
        e = product_entry(p, steps, step_us, None)
        say(f"{p.name}: {step_us:.3f} us per launch, frac {e['roofline']['frac']}")
        strips.append(e)
        p.free()

    value = head.bytes / h_step / 1e3
    ach = value
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h_step / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": head_wl.name, "M": head_wl.M, "K": head_wl.K, "N": head_wl.N, "bits": head_wl.bits,
            "group_size": head_wl.group_size, "seed": head_wl.seed, "weight_copies_rotated": head.R,
            "algorithmic_bytes_per_step": head.bytes, "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "timing": "the timed steps as graph nodes behind a lead-in, minus the lead-in alone, events on the "
                      "launch stream, median of three; cold weights (rotated copies over 512 MiB, caches evicted "
                      "before each replay)",
            "plan": head.plan,
            "weight_layout": "16-column strips (qmm_to_strips once at load time; the same packed words, "
                             "qmm_gemv_ex with QMM_STRIPS)",
            "k_major_us_per_launch": next(e["us_per_launch"] for e in configs if e["workload"] == head_wl.name),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic(head.name, "gemv", head_wl.bits),
            "kernel": head.kernel_name(), "us_per_launch": round(h_step, 3),
            "duration_from": "events on the launch stream around the graph replays (one kernel node per step; "
                             "the replay with the timed steps minus the one without), divided by the steps",
        },
        "configs": configs,
        "strips": strips,
    }
    if not args.no_extras:
        c5 = datagen.WORKLOADS[datagen.HEADLINE_GEMM]
        p = Product(w, torch, datagen, c5.M, c5.K, c5.N, 4, 128, 0, (0, 15), (0.001, 0.004),
                    name=f"gemm_m{c5.M}_k{c5.K}_n{c5.N}_int4_g128")
        step_us = measure(clock, p, GEMM_STEPS, GEMM_WARMUP)
        out["gemm_int4_g128"] = product_entry(p, GEMM_STEPS, step_us, None)
        p.free()
        bf = {}
        for wl in (head_wl, c5):
            p = workload_product(w, torch, datagen, wl, bf16=True)
            steps, warm = (GEMV_STEPS, 20) if p.gemv else (GEMM_STEPS, GEMM_WARMUP)
            step_us = measure(clock, p, steps, warm)
            bf[wl.name] = product_entry(p, steps, step_us, None)
            p.free()
        out["bf16"] = bf
        out["readme_shapes"] = bench_readme_shapes(w, torch, datagen, clock)
        out["floors"] = bench_floors(torch, clock, probes)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(datagen, head_d, head_wl, args.cpu_seconds)
        if gemm_d is not None:
            out["cpu_baseline_gemm"] = cpu_baseline_gemm(datagen, gemm_d, datagen.WORKLOADS[datagen.HEADLINE_GEMM],
                                                         args.cpu_gemm_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
