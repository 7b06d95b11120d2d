"""Parity at the full workload sizes, in the launch plans the benchmark times.

* The prefill product (M=2048, K=4096, N=14336, 8-bit, one group per column)
  against the oracle on every one of its outputs.
* One-hot activations (x = e_k) select row k of the dequantized weight; with
  integer zero points every kernel forms that row exactly and rounds it once,
  so the outputs must equal the oracle's fp16 rounding bit for bit. This is
  run over every k of K at: the GEMM's 256 x 256 block tile (8-bit with one
  group per column, and 4-bit with groups of 128); the decode product at two
  columns per lane (3-bit, N=6144), at four columns per lane with eight rows
  per call (2-bit, N=11008), and in a plan that splits K over blocks (partial
  sums through the workspace).
* The split-K plan returns the same bits call after call.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the parity tests")
    import weight_only_group_amd as w
    w.library()  # raises if the HIP library is missing
    return w


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _mismatches(got, want):
    bad = np.argwhere(got.view(np.uint16) != want.view(np.uint16))
    return [(int(k), int(n), float(got[k, n]), float(want[k, n])) for k, n in bad[:10]], len(bad)


def test_prefill_workload_all_outputs(gpu):
    wl = datagen.WORKLOADS[datagen.HEADLINE_GEMM]
    p = gpu.gemm_plan_info(wl.M, wl.K, wl.N, wl.bits, wl.group_size)
    _say(f"workload {wl.name}: all {wl.M * wl.N} outputs, plan {p}")
    assert (p["bm"], p["bn"]) == (256, 256)
    d = datagen.generate(wl)
    qw, qlo = gpu.qmm_pack(_t(d["codes"]), wl.bits)
    y = gpu.qmm_gemm(_t(d["x"]), qw, qlo, _t(d["zeros"]), _t(d["scales"]), wl.bits, wl.group_size).cpu().numpy()
    y_ref, a = oracle.quantized_matmul_codes(d["x"], d["codes"], d["zeros"], d["scales"], wl.group_size)
    rep = oracle.parity_report(y, y_ref, a)
    _say(f"  max|err|/bound={rep['max_ratio']:.4f} median={rep['median_ratio']:.5f} violations={rep['violations']}")
    assert rep["ok"] and rep["max_ratio"] < 0.35, rep


@pytest.mark.parametrize("bits,gs,zr", [(8, -1, (96, 160)), (4, 128, (0, 15))], ids=["int8_gchan", "int4_g128"])
def test_gemm_one_hot_every_row_at_the_256_tile(gpu, bits, gs, zr):
    K, N = 4096, 14336
    p = gpu.gemm_plan_info(K, K, N, bits, gs)
    _say(f"gemm one-hot K={K} N={N} bits={bits} gs={gs}: plan {p}")
    assert (p["bm"], p["bn"]) == (256, 256)
    d = datagen.small_case(1, K, N, bits, gs, seed=bits + 11, zero_range=zr, scale_range=(0.001, 0.004))
    qw, qlo = gpu.qmm_pack(_t(d["codes"]), bits)
    eye = torch.eye(K, dtype=torch.float16, device=DEV)
    got = gpu.qmm_gemm(eye, qw, qlo, _t(d["zeros"]), _t(d["scales"]), bits, gs).cpu().numpy()
    want = oracle.dequantize_fp16(d["codes"], d["scales"], d["zeros"], gs)
    mism, count = _mismatches(got, want)
    assert count == 0, (count, mism)


# (M, K, N, bits, gs, zero range, plan fields the case must take)
ONE_HOT_GEMV = [
    (1, 2048, 6144, 3, 128, (0, 7), {"kernel": 1, "vec": 2}),      # the 3-bit decode workload
    (8, 4096, 11008, 2, 64, (0, 3), {"kernel": 1, "vec": 4}),      # the 2-bit small-batch workload
    (1, 4096, 4096, 4, 128, (0, 15), {"kernel": 1, "vec": 1}),     # the headline decode workload
    (1, 4096, 1024, 4, 128, (0, 15), {"kernel": 0}),               # narrow: split along K
    (4, 8192, 512, 8, -1, (96, 160), {"kernel": 0}),
]


@pytest.mark.parametrize("M,K,N,bits,gs,zr,want_plan", ONE_HOT_GEMV,
                         ids=[f"m{c[0]}_k{c[1]}_n{c[2]}_b{c[3]}_g{c[4]}" for c in ONE_HOT_GEMV])
def test_gemv_one_hot_every_row(gpu, M, K, N, bits, gs, zr, want_plan):
    p = gpu.gemv_plan_info(M, K, N, bits, gs)
    _say(f"gemv one-hot M={M} K={K} N={N} bits={bits} gs={gs}: plan {p}")
    for f, v in want_plan.items():
        assert p[f] == v, (f, p)
    if want_plan["kernel"] == 0:
        assert p["ksplit"] > 1, p
    d = datagen.small_case(M, K, N, bits, gs, seed=K + N + bits, zero_range=zr)
    qw, qlo = gpu.qmm_pack(_t(d["codes"]), bits)
    z, s = _t(d["zeros"]), _t(d["scales"])
    eye = torch.eye(K, dtype=torch.float16, device=DEV)
    out = torch.empty((K, N), dtype=torch.float16, device=DEV)
    for k0 in range(0, K, M):  # M one-hot rows per call, in the plan above
        gpu.qmm_gemv(eye[k0:k0 + M], qw, qlo, z, s, bits, gs, out=out[k0:k0 + M])
    got = out.cpu().numpy()
    want = oracle.dequantize_fp16(d["codes"], d["scales"], d["zeros"], gs)
    mism, count = _mismatches(got, want)
    assert count == 0, (count, mism)


def test_split_k_plan_is_deterministic(gpu):
    M, K, N, bits, gs = 2, 4096, 1024, 4, 128
    p = gpu.gemv_plan_info(M, K, N, bits, gs)
    assert p["kernel"] == 0 and p["ksplit"] > 1, p
    d = datagen.small_case(M, K, N, bits, gs, seed=3)
    qw, qlo = gpu.qmm_pack(_t(d["codes"]), bits)
    g = {k: _t(d[k]) for k in ("x", "zeros", "scales")}
    outs = [gpu.qmm_gemv(g["x"], qw, qlo, g["zeros"], g["scales"], bits, gs).cpu().numpy() for _ in range(5)]
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16))
    y_ref, a = oracle.quantized_matmul_codes(d["x"], d["codes"], d["zeros"], d["scales"], gs)
    rep = oracle.parity_report(outs[0], y_ref, a)
    assert rep["ok"] and rep["max_ratio"] < 0.35, rep
