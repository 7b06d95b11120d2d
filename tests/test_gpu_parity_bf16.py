"""Parity of the bf16 entry points (x, zero points, scales, bias and output in
bfloat16) with the CPU oracle, through the C ABI.

The oracle takes the bf16 inputs decoded exactly to float64. Products must
satisfy, element by element, |y - y_ref| <= 9e-3 * sum_k |x_k w_kn| + 1e-3
(oracle.REL_TOL_BF16: the dequantized weight and the output are each rounded
once to bf16, relative error up to 2^-8 each, and the fp32 sum adds K * 2^-24).
One-hot activations select single rows of the dequantized weight, which the
kernels form exactly in fp32 and round once: those outputs equal the oracle's
bf16 rounding bit for bit. qmm_dequant_bf16 is bit-exact everywhere.
"""
import json
import os
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


def _bf(bits_u16):
    """bf16 bit patterns (numpy uint16) -> a bfloat16 tensor on the GPU."""
    a = np.ascontiguousarray(np.asarray(bits_u16, dtype=np.uint16)).view(np.int16)
    return torch.from_numpy(a).view(torch.bfloat16).to(DEV)


def _bits(t):
    """A bfloat16 tensor -> its bit patterns (numpy uint16)."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _case(M, K, N, bits, gs, seed, zero_range=None, scale_range=(0.005, 0.05)):
    d = datagen.small_case(M, K, N, bits, gs, seed=seed, zero_range=zero_range, scale_range=scale_range)
    return datagen.as_bf16_case(d)


def _ref(b, gs, bias=None):
    """float64 reference (y, a) from bf16 inputs decoded exactly."""
    return oracle.quantized_matmul_codes(oracle.bf16_to_f64(b["x"]), b["codes"], oracle.bf16_to_f64(b["zeros"]),
                                         oracle.bf16_to_f64(b["scales"]), gs,
                                         bias=None if bias is None else oracle.bf16_to_f64(bias))


def _device(gpu, b, bits):
    qw, qlo = gpu.qmm_pack(torch.from_numpy(np.ascontiguousarray(b["codes"])).to(DEV), bits)
    return qw, qlo, _bf(b["zeros"]), _bf(b["scales"]), _bf(b["x"])


def _check(y, y_ref, a, label, max_ratio=0.35):
    rep = oracle.parity_report(oracle.bf16_to_f64(_bits(y)), y_ref, a, rel_tol=oracle.REL_TOL_BF16)
    _say(f"  {label}: max|err|/bound={rep['max_ratio']:.4f} median={rep['median_ratio']:.5f} "
         f"violations={rep['violations']} nonfinite={rep['nonfinite']}")
    assert rep["ok"], (label, rep)
    assert rep["max_ratio"] < max_ratio, (label, rep)


def _product(gpu, path, *args, **kw):
    return (gpu.qmm_gemv if path == "gemv" else gpu.qmm_gemm)(*args, **kw)


def _run(gpu, path, M, K, N, bits, gs, seed, **kw):
    b = _case(M, K, N, bits, gs, seed, **kw)
    qw, qlo, z, s, x = _device(gpu, b, bits)
    y = _product(gpu, path, x, qw, qlo, z, s, bits, gs)
    assert y.dtype == torch.bfloat16
    return y, b


SWEEP_GEMV = [
    (1, 256, 64, 4, 128), (3, 1024, 264, 4, 64), (16, 256, 520, 4, -1), (5, 512, 136, 8, 128),
    (8, 1024, 8, 8, -1), (8, 256, 264, 2, 32), (2, 256, 200, 3, 32), (8, 1024, 520, 3, 64),
    (1, 96, 24, 3, -1), (4, 512, 200, 1, 32), (16, 1024, 136, 1, -1), (3, 8192, 64, 4, 128),
]


@pytest.mark.parametrize("M,K,N,bits,gs", SWEEP_GEMV)
def test_gemv_bf16_sweep(gpu, M, K, N, bits, gs):
    _say(f"gemv bf16 M={M} K={K} N={N} bits={bits} gs={gs}")
    y, b = _run(gpu, "gemv", M, K, N, bits, gs, seed=M * 7 + K + N)
    _check(y, *_ref(b, gs), "gemv bf16")


SWEEP_GEMM = [
    (1, 256, 64, 4, 128), (17, 512, 264, 4, 64), (300, 256, 520, 4, -1), (257, 320, 264, 4, 32),
    (100, 512, 136, 8, 128), (260, 1024, 264, 8, -1), (64, 96, 8, 8, 32), (270, 256, 264, 2, 32),
    (300, 256, 520, 3, 32), (8, 1024, 40, 3, -1), (70, 512, 264, 1, 64), (260, 288, 520, 1, -1),
    # six K groups of two waves (small grids, long K), one with a K tail
    (100, 2080, 200, 8, 32), (300, 4096, 264, 3, -1),
]


@pytest.mark.parametrize("M,K,N,bits,gs", SWEEP_GEMM)
def test_gemm_bf16_sweep(gpu, M, K, N, bits, gs):
    _say(f"gemm bf16 M={M} K={K} N={N} bits={bits} gs={gs}")
    y, b = _run(gpu, "gemm", M, K, N, bits, gs, seed=M * 5 + K + N)
    _check(y, *_ref(b, gs), "gemm bf16")


# The README's benchmark shapes (M, N, K), 4-bit, group size 128, and one
# that takes the 128 x 128 block tile.
@pytest.mark.parametrize("M,N,K", [(128, 512, 1024), (512, 2048, 4096), (1024, 4096, 256)])
def test_gemm_bf16_mid_m_shapes(gpu, M, N, K):
    _say(f"gemm bf16 mid-M M={M} N={N} K={K}")
    y, b = _run(gpu, "gemm", M, K, N, 4, 128, seed=M + N + K)
    _check(y, *_ref(b, 128), "gemm bf16 mid-M")


def test_gemm_bf16_large_tile(gpu):
    """A product wide enough for the 256 x 256 block tile, 8-bit, one group per column."""
    M, K, N = 2048, 512, 2048
    _say(f"gemm bf16 large tile M={M} K={K} N={N}")
    y, b = _run(gpu, "gemm", M, K, N, 8, -1, seed=11, zero_range=(96, 160), scale_range=(0.001, 0.004))
    _check(y, *_ref(b, -1), "gemm bf16 large tile")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("bits,gs", [(1, 64), (3, 64), (4, 64), (8, 64), (8, -1)])
def test_bf16_non_integer_zero_points(gpu, path, bits, gs):
    M = 4 if path == "gemv" else 70
    _say(f"{path} bf16 non-integer zeros bits={bits} gs={gs}")
    b = _case(M, 512, 264, bits, gs, seed=bits)
    rng = np.random.default_rng(bits + 31)
    b["zeros"] = datagen.round_to_bf16(rng.uniform(-1.5, (1 << bits) + 0.5, size=b["zeros"].shape))
    qw, qlo, z, s, x = _device(gpu, b, bits)
    y = _product(gpu, path, x, qw, qlo, z, s, bits, gs)
    _check(y, *_ref(b, gs), f"{path} bf16 nonint-z")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("bits,gs", [(2, 32), (3, 64), (4, 128), (8, -1), (1, -1)])
def test_bf16_one_hot_rows_bit_exact(gpu, path, bits, gs):
    """x = e_k gives y = bf16(w[k, :]), the oracle's once-rounded dequantized row."""
    K, N = 256, 136
    b = _case(1, K, N, bits, gs, seed=bits * 5 + (gs if gs > 0 else 3))
    qw, qlo, z, s, _ = _device(gpu, b, bits)
    rows = K if gs == -1 else gs
    eps = 16 if bits == 3 else 32 // bits
    probe = sorted(set(list(range(0, 2 * max(eps, 32))) + [g0 * rows for g0 in range(K // rows)] +
                       [g0 * rows + rows - 1 for g0 in range(K // rows)] + [K - 1]))
    _say(f"bf16 one-hot {path} bits={bits} gs={gs}: {len(probe)} rows")
    X = np.zeros((len(probe), K), dtype=np.uint16)
    for i, k in enumerate(probe):
        X[i, k] = 0x3F80  # 1.0
    want = oracle.dequantize_bf16(b["codes"], b["scales"], b["zeros"], gs)[probe]
    if path == "gemv":
        got = np.concatenate([_bits(gpu.qmm_gemv(_bf(X[c:c + 16]), qw, qlo, z, s, bits, gs))
                              for c in range(0, len(probe), 16)])
    else:
        got = _bits(gpu.qmm_gemm(_bf(X), qw, qlo, z, s, bits, gs))
    mism = np.argwhere(got != want)
    assert mism.size == 0, [(probe[i], n, hex(got[i, n]), hex(want[i, n])) for i, n in mism[:10]]


@pytest.mark.parametrize("path,M,K,N,bits,gs", [
    ("gemv", 1, 512, 256, 4, 128),
    ("gemv", 3, 8192, 64, 4, 128),
    ("gemm", 70, 288, 520, 8, -1),
    ("gemm", 300, 512, 264, 3, 64),
])
def test_bf16_bias(gpu, path, M, K, N, bits, gs):
    _say(f"bf16 bias {path} M={M} K={K} N={N} bits={bits} gs={gs}")
    b = _case(M, K, N, bits, gs, seed=M + K + N)
    bias = datagen.round_to_bf16(np.random.default_rng(M).uniform(-4, 4, size=N))
    qw, qlo, z, s, x = _device(gpu, b, bits)
    y = _product(gpu, path, x, qw, qlo, z, s, bits, gs, bias=_bf(bias))
    _check(y, *_ref(b, gs, bias=bias), f"{path} bf16 bias")
    y0 = _product(gpu, path, torch.zeros_like(x), qw, qlo, z, s, bits, gs, bias=_bf(bias))
    assert np.array_equal(_bits(y0), np.tile(bias, (M, 1)))


@pytest.mark.parametrize("bits,K,N,gs", [(1, 256, 72, 32), (2, 512, 136, 64), (3, 256, 200, -1),
                                         (4, 1024, 264, 128), (8, 512, 520, 32)])
@pytest.mark.parametrize("zkind", ["integer", "fractional", "subnormal_scale"])
def test_dequant_bf16_bit_exact(gpu, bits, K, N, gs, zkind):
    _say(f"dequant bf16 bits={bits} K={K} N={N} gs={gs} zeros={zkind}")
    b = _case(1, K, N, bits, gs, seed=K + N + bits)
    if zkind in ("fractional", "subnormal_scale"):
        rng = np.random.default_rng(bits)
        b["zeros"] = datagen.round_to_bf16(rng.uniform(-1.5, (1 << bits) + 0.5, size=b["zeros"].shape))
    if zkind == "subnormal_scale":
        # scales around 2^-136 .. 2^-128 (bf16 subnormals and the lowest normals): the products
        # s * (q - z) fall below 2^-126, where bf16 has the fixed spacing 2^-133
        rng = np.random.default_rng(100 + bits)
        mag = np.ldexp(rng.uniform(1.0, 2.0, size=b["scales"].shape), rng.integers(-136, -128, size=b["scales"].shape))
        b["scales"] = datagen.round_to_bf16(mag.astype(np.float32))
    want = oracle.dequantize_bf16(b["codes"], b["scales"], b["zeros"], gs)
    qw, qlo, z, s, _ = _device(gpu, b, bits)
    w = gpu.qmm_dequant(qw, qlo, z, s, K, bits, gs)
    assert w.dtype == torch.bfloat16
    got = _bits(w)
    mism = np.argwhere(got != want)
    assert mism.size == 0, [(k, n, hex(got[k, n]), hex(want[k, n])) for k, n in mism[:10]]


def test_dequant_bf16_rounding_ties():
    """The hand-worked bf16 cases of tests/golden/dequant_examples.json, on the GPU."""
    import weight_only_group_amd as w
    with open(os.path.join(os.path.dirname(__file__), "golden", "dequant_examples.json")) as f:
        cases = json.load(f)["bf16_dequant_cases"]
    K, N = 32, 8 * len(cases)
    codes = np.zeros((K, N), dtype=np.uint8)
    s = np.zeros((1, N), dtype=np.uint16)
    z = np.zeros((1, N), dtype=np.uint16)
    for i, c in enumerate(cases):
        codes[:, 8 * i:8 * i + 8] = c["q"]
        s[0, 8 * i:8 * i + 8] = int(c["scale_bits"], 16)
        z[0, 8 * i:8 * i + 8] = datagen.round_to_bf16(np.float32(c["zero"]))
    qw, _ = w.qmm_pack(torch.from_numpy(codes).to(DEV), 8)
    got = _bits(w.qmm_dequant(qw, None, _bf(z), _bf(s), K, 8, -1))
    for i, c in enumerate(cases):
        assert np.all(got[:, 8 * i:8 * i + 8] == int(c["bf16_bits"], 16)), c["name"]


@pytest.mark.parametrize("name", [n for n, wl in datagen.WORKLOADS.items() if wl.M <= 16])
def test_workload_bf16_gemv_full(gpu, name):
    wl = datagen.WORKLOADS[name]
    _say(f"workload {name} bf16 (full output)")
    b = datagen.as_bf16_case(datagen.generate(wl))
    qw, qlo, z, s, x = _device(gpu, b, wl.bits)
    y_ref, a = _ref(b, wl.group_size)
    _check(gpu.qmm_gemv(x, qw, qlo, z, s, wl.bits, wl.group_size), y_ref, a, name + " bf16")
    _check(gpu.qmm_gemm(x, qw, qlo, z, s, wl.bits, wl.group_size), y_ref, a, name + " bf16 via gemm")


def test_workload_bf16_prefill_sampled_rows(gpu):
    """The prefill product at full size in bf16; sampled rows against the oracle."""
    wl = datagen.WORKLOADS["gemm_m2048_k4096_n14336_int8_gchan"]
    _say(f"workload {wl.name} bf16 (sampled rows)")
    b = datagen.as_bf16_case(datagen.generate(wl))
    qw, qlo, z, s, x = _device(gpu, b, wl.bits)
    y = gpu.qmm_gemm(x, qw, qlo, z, s, wl.bits, wl.group_size)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float()).all())
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 1023, 2047], rng.choice(wl.M, 58, replace=False)]))
    y_rows = y[torch.as_tensor(rows, device=DEV)]
    sub = dict(b, x=b["x"][rows])
    _check(y_rows, *_ref(sub, wl.group_size), f"{wl.name} bf16 rows={len(rows)}")


def test_bf16_is_deterministic(gpu):
    b = _case(300, 512, 520, 8, -1, seed=3, zero_range=(96, 160))
    qw, qlo, z, s, x = _device(gpu, b, 8)
    r = [_bits(gpu.qmm_gemm(x, qw, qlo, z, s, 8, -1)) for _ in range(2)]
    assert np.array_equal(r[0], r[1])
    b = _case(4, 4096, 256, 4, 128, seed=4)
    qw, qlo, z, s, x = _device(gpu, b, 4)
    r = [_bits(gpu.qmm_gemv(x, qw, qlo, z, s, 4, 128)) for _ in range(3)]
    assert np.array_equal(r[0], r[1]) and np.array_equal(r[0], r[2])


def test_mixed_dtypes_are_refused(gpu):
    b = _case(2, 256, 64, 4, 128, seed=1)
    qw, qlo, z, s, x = _device(gpu, b, 4)
    with pytest.raises(TypeError):
        gpu.qmm_gemv(x, qw, qlo, z.to(torch.float16), s, 4, 128)
    with pytest.raises(TypeError):
        gpu.qmm_gemm(x.to(torch.float16), qw, qlo, z, s, 4, 128)
    with pytest.raises(TypeError):
        gpu.qmm_gemm(x, qw, qlo, z, s, 4, 128, bias=torch.zeros(64, dtype=torch.float16, device=DEV))
