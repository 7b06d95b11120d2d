#!/usr/bin/env python3
"""Throughput of the weight-only group-quantized matmul on one MI355X.

One step is one decode product y = x @ dequant(W) at M=1, K=4096, N=4096,
4-bit codes, group size 128 (one transformer projection), on seeded synthetic
inputs already resident in HBM. The value is achieved HBM bandwidth in GB/s
counting the algorithmic bytes (packed words, scales, zeros, x, y).

Cold cache: every step reads a different copy of the weights, and the copies
together exceed twice the 256 MB Infinity Cache, so each step streams its
weights from HBM. The K timed steps are one HIP graph replay (one kernel node
per step), so host launch overhead is outside the timed region but each
node's dispatch is inside it.

The JSON line also carries:
  roofline      the GEMV kernel against 8 TB/s: algorithmic bytes per launch
                over its average launch duration, taken from events on the
                launch stream around the timed region (the launches run back
                to back, one kernel per step); `traffic` is the HBM bytes the
                FETCH_SIZE / WRITE_SIZE counters saw per launch, each scaled by
                what it reads for a copy of known size (from the committed
                profile summary, null if the kernel source changed)
  cpu_baseline  the CPU oracle on the same workload on this host
  gemm          the prefill product M=2048, K=4096, N=14336, 8-bit, one group
                per column: TFLOP/s against the 2.5 PFLOP/s fp16 dense peak
  readme_shapes the prefill kernel at the README's own benchmark shapes
                (128x512x1024, 256x1024x2048, 512x2048x4096; 4-bit g128), cold
  bf16          the decode and prefill products again with bf16 activations,
                scales, zero points and output (the _bf16 entry points)
  gptq_convert  the load-time conversions of GPTQModel-format inputs: 3-bit
                words of 10 codes to the two 3-bit planes (K=2048, N=6144) and
                packed zero points to (G, N) fp16 (G=64, N=11008), back to back
  floors        reference kernels timed the same way: an empty kernel as a
                graph node, a plain streaming read of the decode product's
                byte count (cold), a long streaming read, a dense MFMA loop
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_DENSE_PEAK_TFLOPS = 2500.0
COLD_BYTES = 512 * 1024 * 1024  # twice the Infinity Cache
METRIC = "M=1 GEMV achieved HBM GB/s (% of peak); M=2048 GEMM TOPS (% MFMA peak)"


def algorithmic_bytes(wl) -> int:
    words = wl.K * wl.N * wl.bits // 8
    sz = 2 * wl.groups * wl.N * 2
    return words + sz + wl.M * wl.K * 2 + wl.M * wl.N * 2


def kernel_source_hash(name: str) -> str:
    p = os.path.join(ROOT, "weight_only_group_amd", "csrc", name)
    h = hashlib.sha256()
    for f in (p, os.path.join(ROOT, "weight_only_group_amd", "csrc", "common.h")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kind: str):
    """HBM bytes per launch from profiles/traffic_<kind>.txt, if taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}.txt")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.loads("".join(line for line in f if not line.startswith("#")))
    except (ValueError, OSError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(rec.get("source", "")):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return 1


def device_inputs(torch, datagen, d, bf16: bool, dev):
    """x, zeros, scales of one case on the GPU, as fp16 or as bf16 (the same draws re-rounded)."""
    if not bf16:
        return tuple(torch.from_numpy(d[k]).to(dev) for k in ("x", "zeros", "scales"))
    b = datagen.as_bf16_case(d)
    return tuple(torch.from_numpy(b[k].view("int16")).view(torch.bfloat16).to(dev) for k in ("x", "zeros", "scales"))


def bench_gemv(w, torch, datagen, steps: int, warmup: int, bf16: bool = False):
    wl = datagen.WORKLOADS[datagen.HEADLINE_GEMV]
    dev = torch.device("cuda:0")
    d = datagen.generate(wl)
    x, z0, s0 = device_inputs(torch, datagen, d, bf16, dev)
    qw0, qlo0 = w.qmm_pack(torch.from_numpy(d["codes"]).to(dev), wl.bits)
    per_copy = qw0.nbytes + z0.nbytes + s0.nbytes + (qlo0.nbytes if qlo0 is not None else 0)
    R = max(1, math.ceil(COLD_BYTES / per_copy))
    copies = [(qw0, qlo0, z0, s0)] + [
        (qw0.clone(), None if qlo0 is None else qlo0.clone(), z0.clone(), s0.clone()) for _ in range(R - 1)]
    y = torch.empty((wl.M, wl.N), dtype=x.dtype, device=dev)
    nbytes = w.workspace_bytes(wl.M, wl.K, wl.N, wl.bits, wl.group_size)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    lib = w.library()
    gemv = lib.qmm_gemv_bf16 if bf16 else lib.qmm_gemv

    def launch(i: int, stream_ptr: int):
        qw, qlo, z, s = copies[i % R]
        st = gemv(x.data_ptr(), wl.M, wl.K, qw.data_ptr(), None if qlo is None else qlo.data_ptr(),
                          z.data_ptr(), s.data_ptr(), None, wl.N, wl.bits, wl.group_size, y.data_ptr(), ws.data_ptr(),
                          ws.numel(), stream_ptr)
        if st != 0:
            raise RuntimeError(f"qmm_gemv failed: {lib.qmm_last_error().decode()}")

    # eager warm-up (also loads the code object)
    cur = torch.cuda.current_stream().cuda_stream
    for i in range(max(warmup, 3)):
        launch(i, cur)
    torch.cuda.synchronize()

    def capture(n: int, offset: int):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sp = torch.cuda.current_stream().cuda_stream
            for i in range(n):
                launch(offset + i, sp)
        return g

    g_warm = capture(max(warmup, 1), 0)
    g_timed = capture(steps, warmup)
    g_warm.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)

    # parity spot check of the last output against the oracle-free invariant: finite
    assert bool(torch.isfinite(y).all())
    return {
        "wl": wl, "R": R, "total_ms": total_ms, "ms_per_step": total_ms / steps,
        "bytes": algorithmic_bytes(wl), "mean_launch_us": total_ms * 1e3 / steps, "d": d, "ws_bytes": nbytes,
    }


def bench_gemm(w, torch, datagen, steps: int, warmup: int, bf16: bool = False):
    wl = datagen.WORKLOADS[datagen.HEADLINE_GEMM]
    dev = torch.device("cuda:0")
    d = datagen.generate(wl)
    x, z0, s0 = device_inputs(torch, datagen, d, bf16, dev)
    qw0, _ = w.qmm_pack(torch.from_numpy(d["codes"]).to(dev), wl.bits)
    R = 4  # weight copies rotated (235 MB of packed weights)
    copies = [(qw0, z0, s0)] + [(qw0.clone(), z0.clone(), s0.clone()) for _ in range(R - 1)]
    y = torch.empty((wl.M, wl.N), dtype=x.dtype, device=dev)
    lib = w.library()
    gemm = lib.qmm_gemm_bf16 if bf16 else lib.qmm_gemm

    def launch(i: int):
        qw, z, s = copies[i % R]
        st = gemm(x.data_ptr(), wl.M, wl.K, qw.data_ptr(), None, z.data_ptr(), s.data_ptr(), None, wl.N, wl.bits,
                  wl.group_size, y.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"qmm_gemm failed: {lib.qmm_last_error().decode()}")

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    # Launches are queued back to back on the current stream; the events on
    # that stream bracket the timed region and its average launch duration.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        launch(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    assert bool(torch.isfinite(y).all())
    flops = 2.0 * wl.M * wl.N * wl.K
    mean_ms = total_ms / steps
    return {"wl": wl, "total_ms": total_ms, "ms_per_step": total_ms / steps, "mean_launch_ms": mean_ms,
            "flops": flops, "bytes": algorithmic_bytes(wl), "d": d}


# The README's benchmark shapes (M, N, K) and the latencies it quotes for them on
# an A100 (4-bit, group size 128 assumed from its quick start; context only: other
# hardware, and the page's latencies and TOPS figures disagree with each other).
README_SHAPES = ((128, 512, 1024, 2.5), (256, 1024, 2048, 8.2), (512, 2048, 4096, 31.5))


def bench_readme_shapes(w, torch, datagen, steps: int = 200):
    """The prefill kernel at the README's own shapes, 4-bit g128, cold weights, graph replay."""
    dev = torch.device("cuda:0")
    lib = w.library()
    out = []
    for M, N, K, page_ms in README_SHAPES:
        d = datagen.small_case(M, K, N, 4, 128, seed=M + N + K)
        x = torch.from_numpy(d["x"]).to(dev)
        z0 = torch.from_numpy(d["zeros"]).to(dev)
        s0 = torch.from_numpy(d["scales"]).to(dev)
        qw0, _ = w.qmm_pack(torch.from_numpy(d["codes"]).to(dev), 4)
        R = max(1, math.ceil(COLD_BYTES / (qw0.nbytes + z0.nbytes + s0.nbytes)))
        copies = [(qw0, z0, s0)] + [(qw0.clone(), z0.clone(), s0.clone()) for _ in range(R - 1)]
        y = torch.empty((M, N), dtype=torch.float16, device=dev)

        def launch(i, sp):
            qw, z, s = copies[i % R]
            st = lib.qmm_gemm(x.data_ptr(), M, K, qw.data_ptr(), None, z.data_ptr(), s.data_ptr(), None, N, 4, 128,
                              y.data_ptr(), sp)
            if st != 0:
                raise RuntimeError(f"qmm_gemm failed: {lib.qmm_last_error().decode()}")

        for i in range(3):
            launch(i, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sp = torch.cuda.current_stream().cuda_stream
            for i in range(steps):
                launch(i, sp)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        out.append({"M": M, "N": N, "K": K, "bits": 4, "group_size": 128, "us": round(us, 3),
                    "TFLOP/s": round(2.0 * M * N * K / us / 1e6, 2), "page_context_a100_ms": page_ms})
        del copies, g
    return out


def bench_gptq_convert(w, torch, datagen, steps: int = 50):
    """The load-time conversions of GPTQModel-format inputs, back-to-back launches between events:
    bytes read and written per launch over the mean launch time. The packed inputs are random
    32-bit words (every pattern is a valid input; the work does not depend on the values)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)

    def words(rows, cols):
        return torch.randint(-2**31, 2**31 - 1, (rows, cols), dtype=torch.int32, device=dev, generator=gen)

    lib = w.library()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(launch):
        for _ in range(5):
            launch()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            launch()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    out = {}
    K, N = 2048, 6144
    w10 = words((K + 9) // 10, N)
    qw = torch.empty((K // 16, N), dtype=torch.int32, device=dev)
    qlo = torch.empty((K // 32, N), dtype=torch.int32, device=dev)

    def repack():
        sp = torch.cuda.current_stream().cuda_stream
        if lib.qmm_repack_3bit10(w10.data_ptr(), K, N, qw.data_ptr(), qlo.data_ptr(), sp) != 0:
            raise RuntimeError(lib.qmm_last_error().decode())

    us = timed(repack)
    nbytes = w10.nbytes + qw.nbytes + qlo.nbytes
    out["repack_3bit10"] = {"K": K, "N": N, "us": round(us, 3), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 1)}
    G, N, bits = 64, 11008, 2
    qz = words(G, (N + 15) // 16)
    zeros = torch.empty((G, N), dtype=torch.float16, device=dev)

    def unpack():
        sp = torch.cuda.current_stream().cuda_stream
        if lib.qmm_unpack_qzeros(qz.data_ptr(), G, N, bits, zeros.data_ptr(), sp) != 0:
            raise RuntimeError(lib.qmm_last_error().decode())

    us = timed(unpack)
    nbytes = qz.nbytes + zeros.nbytes
    out["unpack_qzeros"] = {"G": G, "N": N, "bits": bits, "us": round(us, 3), "bytes": nbytes,
                            "GB/s": round(nbytes / us / 1e3, 1)}
    return out


def floors(torch, gemv_bytes: int):
    """Reference kernels from libqmm_probes.so, timed like the products: the dispatch floor of a
    graph node, a plain streaming read of the decode product's byte count (cold, best of a few
    launch shapes), a long streaming read, and a dense MFMA loop."""
    import ctypes
    path = os.path.join(ROOT, "weight_only_group_amd", "libqmm_probes.so")
    lib = ctypes.CDLL(path)
    lib.qmm_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.qmm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.qmm_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    nbytes = gemv_bytes // 256 * 256
    R = max(1, math.ceil(COLD_BYTES / nbytes))
    buf = torch.empty(R * nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)

    def graph_us(fn, n=400):
        fn(0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sp = torch.cuda.current_stream().cuda_stream
            for i in range(n):
                fn(i, sp)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def ok(st):
        if st != 0:
            raise RuntimeError(f"probe failed with status {st}")

    out = {}
    out["empty_kernel_graph_node_us"] = round(graph_us(lambda i, sp: ok(lib.qmm_probe_empty(256, 1024, sp))), 3)
    best = None
    for blocks, threads in ((256, 1024), (512, 1024), (1024, 512), (2048, 256)):
        us = graph_us(lambda i, sp: ok(lib.qmm_probe_read(buf.data_ptr() + (i % R) * nbytes, nbytes, blocks, threads,
                                                          sink.data_ptr(), sp)))
        if best is None or us < best[0]:
            best = (us, blocks, threads)
    out["read_same_bytes_as_decode"] = {"bytes": nbytes, "us": round(best[0], 3),
                                        "GB/s": round(nbytes / best[0] / 1e3, 1), "blocks": best[1],
                                        "threads": best[2], "cold": True}
    big = R * nbytes
    us = graph_us(lambda i, sp: ok(lib.qmm_probe_read(buf.data_ptr(), big, 8192, 512, sink.data_ptr(), sp)), n=20)
    out["read_long"] = {"bytes": big, "us": round(us, 1), "GB/s": round(big / us / 1e3, 1)}
    iters, blocks = 4000, 1024
    us = graph_us(lambda i, sp: ok(lib.qmm_probe_mfma(blocks, iters, sink.data_ptr(), sp)), n=5)
    flops = blocks * 4 * 4 * iters * 2.0 * 32 * 32 * 16
    out["mfma_32x32x16_f16"] = {"TFLOP/s": round(flops / us / 1e6, 1), "blocks": blocks, "iters": iters}
    del buf
    return out


def cpu_baseline_gemv(datagen, d, seconds: float):
    import oracle
    wl = datagen.WORKLOADS[datagen.HEADLINE_GEMV]
    qw, qlo = oracle.pack(d["codes"], wl.bits)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.quantized_matmul(d["x"], qw, qlo, d["zeros"], d["scales"], wl.bits, wl.group_size)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    return {"value": round(algorithmic_bytes(wl) / per / 1e9, 4), "unit": "GB/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"the whole workload ({wl.name}) from packed words: unpack, float64 dequantize and "
                      f"product; {n} calls in {el:.1f} s, {per * 1e3:.1f} ms each"}


def cpu_baseline_gemm(datagen, d, rows: int):
    import oracle
    wl = datagen.WORKLOADS[datagen.HEADLINE_GEMM]
    qw, _ = oracle.pack(d["codes"], wl.bits)
    t0 = time.perf_counter()
    oracle.quantized_matmul(d["x"][:rows], qw, None, d["zeros"], d["scales"], wl.bits, wl.group_size)
    el = time.perf_counter() - t0
    return {"value": round(2.0 * rows * wl.N * wl.K / el / 1e12, 6), "unit": "TFLOP/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"first {rows} of {wl.M} rows of {wl.name} from packed words (unpack, float64 dequantize of "
                      f"the whole weight, product), one call, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500, help="timed decode products")
    ap.add_argument("--warmup", type=int, default=50)
    # Back-to-back prefill launches dip to ~1.25x their time between about the
    # 10th and 40th launch (a clock transient) and settle after ~80; the
    # default warm-up runs past the dip so that the timed launches are at the
    # steady state.
    ap.add_argument("--gemm-steps", type=int, default=40)
    ap.add_argument("--gemm-warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget for the GEMV baseline")
    ap.add_argument("--cpu-gemm-rows", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-floors", action="store_true", help="skip the reference kernels (empty launch, "
                    "streaming read, MFMA loop)")
    ap.add_argument("--no-bf16", action="store_true", help="skip the bf16 products")
    ap.add_argument("--no-gptq", action="store_true", help="skip the GPTQModel-format conversions")
    ap.add_argument("--only", choices=("gemv", "gemm", "gemv_bf16", "gemm_bf16"), default=None,
                    help="run one product only and print its own line (for profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the products, run 4 plain device copies of MIB MiB each (outside every timed "
                         "region) so that a counter profile can scale FETCH_SIZE / WRITE_SIZE by a copy of "
                         "known size")
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


def gemm_line(gm):
    return {"workload": gm["wl"].name, "ms_per_step": round(gm["ms_per_step"], 4),
            "mean_launch_ms": round(gm["mean_launch_ms"], 4),
            "TFLOP/s": round(gm["flops"] / (gm["mean_launch_ms"] * 1e-3) / 1e12, 2)}


def gemv_line(gv):
    return {"workload": gv["wl"].name, "ms_per_step": round(gv["ms_per_step"], 6),
            "GB/s": round(gv["bytes"] / (gv["ms_per_step"] * 1e-3) / 1e9, 2)}


def run(args, torch, datagen, w):
    if args.only in ("gemm", "gemm_bf16"):
        gm = bench_gemm(w, torch, datagen, args.gemm_steps, args.gemm_warmup, bf16=args.only == "gemm_bf16")
        print(json.dumps(dict(gemm_line(gm), dtype="bf16" if args.only == "gemm_bf16" else "f16")), flush=True)
        return
    if args.only == "gemv_bf16":
        gv = bench_gemv(w, torch, datagen, args.steps, args.warmup, bf16=True)
        print(json.dumps(dict(gemv_line(gv), dtype="bf16")), flush=True)
        return
    gv = bench_gemv(w, torch, datagen, args.steps, args.warmup)
    if args.only == "gemv":
        print(json.dumps(dict(gemv_line(gv), dtype="f16")), flush=True)
        return
    wl = gv["wl"]
    value = gv["bytes"] / (gv["ms_per_step"] * 1e-3) / 1e9
    achieved = gv["bytes"] / (gv["mean_launch_us"] * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(gv["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "bits": wl.bits, "group_size": wl.group_size,
            "seed": wl.seed, "weight_copies_rotated": gv["R"], "algorithmic_bytes_per_step": gv["bytes"],
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "timing": "one HIP graph replay of the timed steps, events around it",
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic("gemv"),
            "kernel": "gemv_kernel, 4-bit instance", "mean_launch_us": round(gv["mean_launch_us"], 3),
        },
    }
    if not args.no_gemm:
        gm = bench_gemm(w, torch, datagen, args.gemm_steps, args.gemm_warmup)
        tflops = gm["flops"] / (gm["ms_per_step"] * 1e-3) / 1e12
        k_tflops = gm["flops"] / (gm["mean_launch_ms"] * 1e-3) / 1e12
        out["gemm"] = {
            "workload": gm["wl"].name, "value": round(tflops, 2), "unit": "TFLOP/s",
            "ms_per_step": round(gm["ms_per_step"], 4), "pct_of_fp16_dense_peak": round(100 * tflops / FP16_DENSE_PEAK_TFLOPS, 2),
            "roofline": {"bound": "mfma", "achieved": round(k_tflops, 2), "peak": FP16_DENSE_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(k_tflops / FP16_DENSE_PEAK_TFLOPS, 4),
                         "traffic": committed_traffic("gemm"), "kernel": "gemm_kernel, 8-bit post-scale instance",
                         "mean_launch_ms": round(gm["mean_launch_ms"], 4)},
            "timing": f"{args.gemm_warmup} untimed launches, then {args.gemm_steps} back to back between events",
        }
    if not args.no_gemm:
        out["readme_shapes"] = bench_readme_shapes(w, torch, datagen)
    if not args.no_bf16:
        # bf16 data, same workloads; the bf16 dense MFMA peak equals the fp16 one
        gvb = bench_gemv(w, torch, datagen, args.steps, args.warmup, bf16=True)
        out["bf16"] = {"gemv": dict(gemv_line(gvb), pct_of_hbm_peak=round(
            100 * gvb["bytes"] / (gvb["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2))}
        if not args.no_gemm:
            gmb = bench_gemm(w, torch, datagen, args.gemm_steps, args.gemm_warmup, bf16=True)
            t = gmb["flops"] / (gmb["mean_launch_ms"] * 1e-3) / 1e12
            out["bf16"]["gemm"] = dict(gemm_line(gmb), pct_of_bf16_dense_peak=round(100 * t / FP16_DENSE_PEAK_TFLOPS, 2))
    if not args.no_gptq:
        out["gptq_convert"] = bench_gptq_convert(w, torch, datagen)
    if not args.no_floors:
        out["floors"] = floors(torch, gv["bytes"])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_gemv(datagen, gv["d"], args.cpu_seconds)
        if not args.no_gemm:
            out["gemm"]["cpu_baseline"] = cpu_baseline_gemm(datagen, gm["d"], args.cpu_gemm_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
