"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Packing and unpacking must match bit for bit. Products must satisfy, element
by element, |y - y_ref| <= 2e-3 * sum_k |x_k w_kn| + 1e-3 with y decoded
exactly from fp16. One-hot activations select single rows of the
dequantized weight; those outputs are exact fp16 roundings and must match the
oracle's rounding bit for bit, which pins every index of the kernels.
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


def _t(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def _to_gpu_case(d):
    return {k: _t(v) for k, v in d.items() if not k.endswith("_f32")}


def _pack_gpu(w, codes_np, bits):
    qw, qlo = w.qmm_pack(_t(codes_np), bits)
    return qw, qlo


def _product(w, path, x, qw, qlo, z, s, bits, gs):
    if path == "gemv":
        return w.qmm_gemv(x, qw, qlo, z, s, bits, gs)
    return w.qmm_gemm(x, qw, qlo, z, s, bits, gs)


def _check(y_gpu, y_ref, a, label, max_ratio=0.35):
    rep = oracle.parity_report(y_gpu, y_ref, a)
    _say(f"  {label}: max|err|/bound={rep['max_ratio']:.4f} median={rep['median_ratio']:.5f} "
         f"violations={rep['violations']} nonfinite={rep['nonfinite']}")
    assert rep["ok"], (label, rep)
    # The bound is loose; a sound kernel stays well inside it.
    assert rep["max_ratio"] < max_ratio, (label, rep)


# ------------------------------------------------------------------ packing

PACK_SHAPES = [(32, 8), (64, 24), (96, 520), (512, 256), (256, 1000)]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("K,N", PACK_SHAPES)
def test_pack_unpack_bit_exact(gpu, bits, K, N):
    if K % (32 if bits == 3 else 32 // bits):
        pytest.skip("K not a multiple of the word size")
    _say(f"pack/unpack bits={bits} K={K} N={N}")
    codes = datagen.draw_codes(K, N, bits, seed=K + N + bits)
    qw_ref, qlo_ref = oracle.pack(codes, bits)
    qw, qlo = _pack_gpu(gpu, codes, bits)
    torch.cuda.synchronize()
    assert np.array_equal(qw.cpu().numpy(), qw_ref)
    if bits == 3:
        assert np.array_equal(qlo.cpu().numpy(), qlo_ref)
    back = gpu.qmm_unpack(_t(qw_ref), None if qlo_ref is None else _t(qlo_ref), K, bits)
    assert np.array_equal(back.cpu().numpy(), codes)


@pytest.mark.parametrize("name", list(datagen.WORKLOADS))
def test_pack_workload_shapes_bit_exact(gpu, name):
    wl = datagen.WORKLOADS[name]
    _say(f"pack/unpack workload {name}")
    codes = datagen.draw_codes(wl.K, wl.N, wl.bits, wl.seed)
    qw_ref, qlo_ref = oracle.pack(codes, wl.bits)
    qw, qlo = _pack_gpu(gpu, codes, wl.bits)
    assert np.array_equal(qw.cpu().numpy(), qw_ref)
    if wl.bits == 3:
        assert np.array_equal(qlo.cpu().numpy(), qlo_ref)
    back = gpu.qmm_unpack(qw, qlo, wl.K, wl.bits)
    assert np.array_equal(back.cpu().numpy(), codes)


def test_pack_counts_and_masks_out_of_range_codes(gpu):
    rng = np.random.default_rng(1)
    for bits in (2, 3, 4):
        codes = rng.integers(0, 256, size=(64, 40), dtype=np.uint8)
        qw, qlo, bad = gpu.qmm_pack(_t(codes), bits, count_bad=True)
        qw_ref, qlo_ref = oracle.pack(codes, bits)
        assert np.array_equal(qw.cpu().numpy(), qw_ref)
        if bits == 3:
            assert np.array_equal(qlo.cpu().numpy(), qlo_ref)
        assert int(bad.item()) == oracle.count_out_of_range(codes, bits)


# ------------------------------------------------------------------ products

def _run(gpu, path, M, K, N, bits, gs, seed=0, zero_range=None, nonint_zero=False, scale_range=(0.005, 0.05)):
    d = datagen.small_case(M, K, N, bits, gs, seed=seed, zero_range=zero_range, scale_range=scale_range)
    if nonint_zero:
        rng = np.random.default_rng(seed + 99)
        d["zeros"] = rng.uniform(-1.5, (1 << bits) + 0.5, size=d["zeros"].shape).astype(np.float16)
    qw_ref, qlo_ref = oracle.pack(d["codes"], bits)
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    y = _product(gpu, path, g["x"], qw, qlo, g["zeros"], g["scales"], bits, gs)
    y_ref, a = oracle.quantized_matmul(d["x"], qw_ref, qlo_ref, d["zeros"], d["scales"], bits, gs)
    return y.cpu().numpy(), y_ref, a


SWEEP_GEMV = [
    # (M, K, N, bits, gs): ragged N tails (not multiples of 64), K spanning several units and groups
    (1, 256, 64, 4, 128), (1, 512, 200, 4, 32), (3, 1024, 264, 4, 64), (16, 256, 520, 4, -1),
    (1, 256, 72, 8, 32), (5, 512, 136, 8, 128), (8, 1024, 8, 8, -1),
    (1, 512, 96, 2, 64), (8, 256, 264, 2, 32), (16, 2048, 40, 2, 128),
    (1, 512, 128, 3, 128), (2, 256, 200, 3, 32), (8, 1024, 520, 3, 64), (1, 96, 24, 3, -1),
    (1, 32, 8, 4, 32), (16, 32, 8, 8, -1),
    (1, 256, 64, 1, 128), (4, 512, 200, 1, 32), (16, 1024, 136, 1, -1),
]


@pytest.mark.parametrize("M,K,N,bits,gs", SWEEP_GEMV)
def test_gemv_sweep(gpu, M, K, N, bits, gs):
    _say(f"gemv M={M} K={K} N={N} bits={bits} gs={gs}")
    y, y_ref, a = _run(gpu, "gemv", M, K, N, bits, gs, seed=M * 7 + K + N)
    _check(y, y_ref, a, "gemv")


# Wave-kernel grids around the one-XCD launch: up to 32 strips (one XCD's CUs, the last strip
# ragged in some) run on XCD 0 alone with the other XCDs' workgroups returning at once; 33
# strips take all XCDs. Every output is compared.
ONE_XCD = [
    (1, 512, 504, 4, 128), (1, 512, 512, 8, -1), (8, 512, 512, 2, 64), (16, 512, 504, 3, 32),
    (8, 512, 200, 1, 32), (1, 512, 520, 4, 128), (16, 512, 520, 8, -1),
]


@pytest.mark.parametrize("M,K,N,bits,gs", ONE_XCD)
def test_gemv_one_xcd_boundary(gpu, M, K, N, bits, gs):
    plan = gpu.gemv_plan_info(M, K, N, bits, gs)
    assert plan["kernel"] == 1, plan  # the wave kernel, which holds the one-XCD launch
    assert plan["one_xcd"] == int(plan["strips"] <= plan["cus"] // plan["xcds"]), plan
    _say(f"gemv (one-XCD boundary, {plan['strips']} strips) M={M} K={K} N={N} bits={bits} gs={gs}")
    y, y_ref, a = _run(gpu, "gemv", M, K, N, bits, gs, seed=M + K + N + bits, nonint_zero=True)
    _check(y, y_ref, a, "gemv")


SWEEP_GEMM = [
    (1, 256, 64, 4, 128), (17, 512, 264, 4, 64), (300, 256, 520, 4, -1), (257, 320, 264, 4, 32),
    (100, 512, 136, 8, 128), (260, 1024, 264, 8, -1), (64, 96, 8, 8, 32),
    (33, 512, 96, 2, 64), (270, 256, 264, 2, 32),
    (40, 512, 128, 3, 128), (300, 256, 520, 3, 32), (8, 1024, 40, 3, -1),
    (70, 512, 264, 1, 64), (260, 288, 520, 1, -1),
    # extremes: the smallest legal product (one 32-row unit, 8 columns), a tall one (65536 rows,
    # 256 row tiles in one column tile) and a wide one (65536 columns, one row tile)
    (1, 32, 8, 4, 32), (1, 32, 8, 3, -1), (65536, 64, 8, 4, -1), (16, 32, 65536, 8, 32),
]


@pytest.mark.parametrize("M,K,N,bits,gs", SWEEP_GEMM)
def test_gemm_sweep(gpu, M, K, N, bits, gs):
    _say(f"gemm M={M} K={K} N={N} bits={bits} gs={gs}")
    y, y_ref, a = _run(gpu, "gemm", M, K, N, bits, gs, seed=M * 5 + K + N)
    _check(y, y_ref, a, "gemm")


# The README's benchmark shapes (M, N, K) with its quick-start format (4-bit,
# group size 128), and a shape that takes the 128 x 128 block tile.
README_SHAPES = [(128, 512, 1024), (256, 1024, 2048), (512, 2048, 4096), (1024, 4096, 256)]


@pytest.mark.parametrize("M,N,K", README_SHAPES)
def test_gemm_mid_m_shapes(gpu, M, N, K):
    _say(f"gemm mid-M M={M} N={N} K={K} 4-bit g128")
    y, y_ref, a = _run(gpu, "gemm", M, K, N, 4, 128, seed=M + N + K)
    _check(y, y_ref, a, "gemm mid-M")


# Grids too small for 128 x 128 tiles with K long enough that six K groups of
# two waves give each group a shorter chain of slabs than four groups of four:
# every width, group sizes 32 / 64 / 128 / -1, a K tail (2080 = 32.5 slabs),
# ragged M and N, integer and non-integer zero points.
SIX_GROUPS = [(64, 4096, 136, 2, 64), (100, 2080, 200, 8, 32), (33, 2048, 520, 1, 128), (300, 4096, 264, 3, -1),
              (200, 8192, 72, 4, 128)]


@pytest.mark.parametrize("nonint", [False, True], ids=["intz", "fracz"])
@pytest.mark.parametrize("M,K,N,bits,gs", SIX_GROUPS)
def test_gemm_six_k_groups(gpu, M, K, N, bits, gs, nonint):
    _say(f"gemm six K groups M={M} K={K} N={N} bits={bits} gs={gs} nonint={nonint}")
    y, y_ref, a = _run(gpu, "gemm", M, K, N, bits, gs, seed=M + K + N + bits, nonint_zero=nonint)
    _check(y, y_ref, a, "gemm six K groups")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_non_integer_zero_points(gpu, path, bits):
    _say(f"{path} non-integer zeros bits={bits}")
    M = 4 if path == "gemv" else 70
    y, y_ref, a = _run(gpu, path, M, 512, 264, bits, 64, seed=bits, nonint_zero=True)
    _check(y, y_ref, a, f"{path} nonint-z")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("M,K,N,bits", [(70, 512, 800, 8), (300, 288, 800, 4), (260, 1024, 776, 2), (40, 544, 784, 3)])
def test_one_group_zero_points_mixed(gpu, path, M, K, N, bits):
    """group_size -1 with column blocks of integer zero points, non-integer ones, and integers above 1024
    (where 1024 + z is not an fp16 integer of spacing 1). K = 288 and 544 leave a tail of a 64-row slab."""
    if path == "gemv":
        M = min(M, 16)
    _say(f"{path} one-group mixed zeros M={M} K={K} N={N} bits={bits}")
    d = datagen.small_case(M, K, N, bits, -1, seed=K + N + bits)
    rng = np.random.default_rng(bits + 7)
    z = d["zeros"].astype(np.float64)
    z[:, 256:512] = rng.uniform(-2.0, (1 << bits) + 2.0, size=(1, 256))
    z[:, 512:640] = rng.integers(1025, 1100, size=(1, 128))
    z[:, 640:] = rng.uniform(1024.0, 1030.0, size=(1, N - 640))
    d["zeros"] = z.astype(np.float16)
    qw_ref, qlo_ref = oracle.pack(d["codes"], bits)
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    y = _product(gpu, path, g["x"], qw, qlo, g["zeros"], g["scales"], bits, -1)
    y_ref, a = oracle.quantized_matmul(d["x"], qw_ref, qlo_ref, d["zeros"], d["scales"], bits, -1)
    _check(y.cpu().numpy(), y_ref, a, f"{path} one-group mixed zeros")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("bits,gs", [(2, 32), (3, 64), (4, 128), (8, -1), (4, 32), (1, 32), (1, -1)])
def test_one_hot_rows_bit_exact(gpu, path, bits, gs):
    """x = e_k gives y = fp16(w[k, :]); probes every word slot and the first and last k of each group."""
    K, N = 256, 136
    d = datagen.small_case(1, K, N, bits, gs, seed=bits * 3 + (gs if gs > 0 else 1))
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    g = _to_gpu_case(d)
    rows = K if gs == -1 else gs
    eps = 16 if bits == 3 else 32 // bits
    probe = sorted(set(list(range(0, 2 * max(eps, 32))) + [g0 * rows for g0 in range(K // rows)] +
                       [g0 * rows + rows - 1 for g0 in range(K // rows)] + [K - 1]))
    _say(f"one-hot {path} bits={bits} gs={gs}: {len(probe)} rows")
    # Each probe is one row of x; run up to 16 rows per call on the GEMV, all at once on the GEMM.
    X = np.zeros((len(probe), K), dtype=np.float16)
    for i, k in enumerate(probe):
        X[i, k] = 1
    w_ref = oracle.dequantize(d["codes"], d["scales"], d["zeros"], gs)
    want = w_ref[probe].astype(np.float16)
    got = []
    if path == "gemv":
        for c in range(0, len(probe), 16):
            got.append(gpu.qmm_gemv(_t(X[c:c + 16]), qw, qlo, g["zeros"], g["scales"], bits, gs).cpu().numpy())
        got = np.concatenate(got)
    else:
        got = gpu.qmm_gemm(_t(X), qw, qlo, g["zeros"], g["scales"], bits, gs).cpu().numpy()
    mism = np.argwhere(got.view(np.uint16) != want.view(np.uint16))
    assert mism.size == 0, [(probe[i], n, float(got[i, n]), float(want[i, n])) for i, n in mism[:10]]


# Extreme value regimes for the decode product's subnormal form (codes as fp16
# subnormals, activations prescaled by 2^-e, s and z applied to per-group sums)
# and for the GEMM: activations that are fp16 subnormals or large, zero points
# far outside the code range (negative, above 1024, fractional), scales that
# are fp16 subnormals or large. Each regime keeps y inside the fp16 range.
EXTREME = ("tiny_x", "large_x", "far_zeros", "scale_range")


def _extreme_case(regime, M, K, N, bits, gs, seed):
    rng = np.random.default_rng(seed)
    G = oracle.num_groups(K, gs)
    codes = datagen.draw_codes(K, N, bits, seed=seed)
    x = datagen.draw_x_f32(M, K, seed).astype(np.float64)
    z = rng.integers(0, 1 << bits, size=(G, N)).astype(np.float64)
    s = rng.uniform(0.005, 0.02, size=(G, N))
    if regime == "tiny_x":  # a third of x below the fp16 normal range, some zeros
        sel = rng.random(size=x.shape)
        x = np.where(sel < 0.33, x * 2.0 ** -16, x)
        x[sel > 0.97] = 0.0
    elif regime == "large_x":
        x = x * 200.0
        s = s * 0.05
    elif regime == "far_zeros":  # negative, fractional, above 1024
        kind = rng.integers(0, 3, size=(G, N))
        z = np.where(kind == 0, -rng.uniform(1, 40, size=(G, N)), np.where(kind == 1, rng.uniform(1024, 1500, size=(G, N)), z + 0.37))
        s = s * 0.02
    elif regime == "scale_range":  # fp16 subnormal scales next to large ones
        kind = rng.integers(0, 3, size=(G, N))
        s = np.where(kind == 0, rng.uniform(2.0 ** -24, 2.0 ** -15, size=(G, N)), np.where(kind == 1, rng.uniform(1, 4, size=(G, N)), s))
    return codes, x.astype(np.float16), z.astype(np.float16), s.astype(np.float16)


@pytest.mark.parametrize("regime", EXTREME)
@pytest.mark.parametrize("bits", (1, 2, 3, 4, 8))
def test_extreme_values(gpu, regime, bits):
    cases = [("gemv", 1, 1024, 512, 128), ("gemv", 8, 1024, 528, 64), ("gemm", 96, 1024, 520, 128)]
    for path, M, K, N, gs in cases:
        codes, x, z, s = _extreme_case(regime, M, K, N, bits, gs, seed=31 * bits + M + len(regime))
        _say(f"extreme {regime} {path} M={M} K={K} N={N} bits={bits} gs={gs}")
        qw, qlo = _pack_gpu(gpu, codes, bits)
        y_ref, a = oracle.quantized_matmul_codes(x, codes, z, s, gs)
        assert np.all(np.abs(y_ref) < 6e4), "the case must stay inside the fp16 range"
        y = _product(gpu, path, _t(x), qw, qlo, _t(z), _t(s), bits, gs)
        _check(y.cpu().numpy().astype(np.float64), y_ref, a, f"{regime} {path} bits={bits}")
        if path == "gemv":
            sw = gpu.qmm_to_strips(qw)
            slo = None if qlo is None else gpu.qmm_to_strips(qlo)
            y2 = gpu.qmm_gemv(_t(x), sw, slo, _t(z), _t(s), bits, gs, strips=True)
            _check(y2.cpu().numpy().astype(np.float64), y_ref, a, f"{regime} {path} strips bits={bits}")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_column_sums(gpu, path):
    """x = 1 sums every column of the dequantized weight."""
    K, N, bits, gs = 512, 264, 4, 128
    d = datagen.small_case(2, K, N, bits, gs, seed=21)
    x = np.ones((2, K), dtype=np.float16)
    x[1] = -1
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    g = _to_gpu_case(d)
    y = _product(gpu, path, _t(x), qw, qlo, g["zeros"], g["scales"], bits, gs).cpu().numpy()
    y_ref, a = oracle.quantized_matmul_codes(x, d["codes"], d["zeros"], d["scales"], gs)
    _check(y, y_ref, a, f"{path} column sums")


def test_gemv_is_deterministic_and_reuses_workspace(gpu):
    wl = datagen.WORKLOADS["gemv_m1_k4096_n4096_int4_g128"]
    d = datagen.generate(wl)
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], wl.bits)
    outs = [gpu.qmm_gemv(g["x"], qw, qlo, g["zeros"], g["scales"], wl.bits, wl.group_size).cpu().numpy()
            for _ in range(3)]
    # a different shape through the same cached workspace in between
    d2 = datagen.small_case(3, 1024, 264, 4, 64, seed=5)
    g2 = _to_gpu_case(d2)
    qw2, _ = _pack_gpu(gpu, d2["codes"], 4)
    y2 = gpu.qmm_gemv(g2["x"], qw2, None, g2["zeros"], g2["scales"], 4, 64).cpu().numpy()
    outs.append(gpu.qmm_gemv(g["x"], qw, qlo, g["zeros"], g["scales"], wl.bits, wl.group_size).cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16))
    qw2_ref, _ = oracle.pack(d2["codes"], 4)
    y2_ref, a2 = oracle.quantized_matmul(d2["x"], qw2_ref, None, d2["zeros"], d2["scales"], 4, 64)
    _check(y2, y2_ref, a2, "gemv after reuse")


def test_gemm_is_deterministic(gpu):
    d = datagen.small_case(300, 512, 520, 8, -1, seed=3, zero_range=(96, 160))
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], 8)
    a = gpu.qmm_gemm(g["x"], qw, qlo, g["zeros"], g["scales"], 8, -1).cpu().numpy()
    b = gpu.qmm_gemm(g["x"], qw, qlo, g["zeros"], g["scales"], 8, -1).cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_non_default_stream(gpu):
    d = datagen.small_case(1, 1024, 264, 3, 128, seed=8)
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], 3)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = gpu.qmm_gemv(g["x"], qw, qlo, g["zeros"], g["scales"], 3, 128)
        y2 = gpu.qmm_gemm(g["x"], qw, qlo, g["zeros"], g["scales"], 3, 128)
    s.synchronize()
    qw_ref, qlo_ref = oracle.pack(d["codes"], 3)
    y_ref, a = oracle.quantized_matmul(d["x"], qw_ref, qlo_ref, d["zeros"], d["scales"], 3, 128)
    _check(y.cpu().numpy(), y_ref, a, "gemv side stream")
    _check(y2.cpu().numpy(), y_ref, a, "gemm side stream")


def test_errors_on_device(gpu):
    """Invalid requests are refused on a real device too, and leave the output untouched."""
    import weight_only_group_amd as w
    x = torch.zeros((1, 256), dtype=torch.float16, device=DEV)
    qw = torch.zeros((32, 64), dtype=torch.int32, device=DEV)
    z = torch.zeros((2, 64), dtype=torch.float16, device=DEV)
    y = torch.full((1, 64), 7.0, dtype=torch.float16, device=DEV)
    with pytest.raises(w.QmmError) as e:
        w.qmm_gemv(x, qw, None, z, z, 4, 100, out=y)
    assert e.value.status == 4
    with pytest.raises(w.QmmError) as e:
        w.qmm_gemm(x, qw, None, z, z, 5, 128, out=y)
    assert e.value.status == 2
    lib = w.library()
    st = lib.qmm_gemv(x.data_ptr() + 2, 1, 256, qw.data_ptr(), None, z.data_ptr(), z.data_ptr(), None, 64, 4, 128,
                      y.data_ptr(), None, 0, None)
    assert st == 5
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ------------------------------------------------------------------ dequantize, bias

DEQUANT_CASES = [(1, 256, 72, 32), (2, 512, 136, 64), (3, 256, 200, -1), (4, 1024, 264, 128), (8, 512, 520, 32),
                 (4, 32, 8, -1)]


@pytest.mark.parametrize("bits,K,N,gs", DEQUANT_CASES)
@pytest.mark.parametrize("zkind", ["integer", "fractional"])
def test_dequant_bit_exact(gpu, bits, K, N, gs, zkind):
    """qmm_dequant returns fp16(s * (q - z)) rounded once: equal bit for bit to the oracle."""
    _say(f"dequant bits={bits} K={K} N={N} gs={gs} zeros={zkind}")
    d = datagen.small_case(1, K, N, bits, gs, seed=K + N + bits)
    if zkind == "fractional":
        rng = np.random.default_rng(bits)
        d["zeros"] = rng.uniform(-1.5, (1 << bits) + 0.5, size=d["zeros"].shape).astype(np.float16)
    want = oracle.dequantize_fp16(d["codes"], d["scales"], d["zeros"], gs)
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    g = _to_gpu_case(d)
    got = gpu.qmm_dequant(qw, qlo, g["zeros"], g["scales"], K, bits, gs).cpu().numpy()
    mism = np.argwhere(got.view(np.uint16) != want.view(np.uint16))
    assert mism.size == 0, [(k, n, float(got[k, n]), float(want[k, n])) for k, n in mism[:10]]


def test_dequant_rounding_ties(gpu):
    """The hand-worked ties of tests/golden/dequant_examples.json round to even on the GPU too."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "dequant_examples.json")) as f:
        cases = json.load(f)["fp16_cases"]
    K, N = 32, 8 * len(cases)
    codes = np.zeros((K, N), dtype=np.uint8)
    s = np.zeros((1, N), dtype=np.uint16)
    z = np.zeros((1, N), dtype=np.float16)
    for i, c in enumerate(cases):
        codes[:, 8 * i:8 * i + 8] = c["q"]
        s[0, 8 * i:8 * i + 8] = int(c["scale_bits"], 16)
        z[0, 8 * i:8 * i + 8] = c["zero"]
    qw, _ = _pack_gpu(gpu, codes, 8)
    got = gpu.qmm_dequant(qw, None, _t(z), _t(s.view(np.float16)), K, 8, -1).cpu().numpy().view(np.uint16)
    for i, c in enumerate(cases):
        assert np.all(got[:, 8 * i:8 * i + 8] == int(c["fp16_bits"], 16)), c["name"]


@pytest.mark.parametrize("path,M,K,N,bits,gs", [
    ("gemv", 1, 512, 256, 4, 128),      # one block per strip
    ("gemv", 3, 8192, 64, 4, 128),      # blocks along K hand over through the workspace
    ("gemv", 8, 1024, 520, 1, -1),
    ("gemm", 70, 288, 520, 8, -1),      # K tail, ragged N, scale after the accumulation
    ("gemm", 300, 512, 264, 3, 64),     # scale inside the dequantization
])
def test_bias(gpu, path, M, K, N, bits, gs):
    _say(f"bias {path} M={M} K={K} N={N} bits={bits} gs={gs}")
    d = datagen.small_case(M, K, N, bits, gs, seed=M + K + N)
    b = np.random.default_rng(M).uniform(-4, 4, size=N).astype(np.float16)
    qw_ref, qlo_ref = oracle.pack(d["codes"], bits)
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    g = _to_gpu_case(d)
    fn = gpu.qmm_gemv if path == "gemv" else gpu.qmm_gemm
    y = fn(g["x"], qw, qlo, g["zeros"], g["scales"], bits, gs, bias=_t(b)).cpu().numpy()
    y_ref, a = oracle.quantized_matmul(d["x"], qw_ref, qlo_ref, d["zeros"], d["scales"], bits, gs, bias=b)
    _check(y, y_ref, a, f"{path} bias")
    # x = 0: the output is the bias row, exactly
    y0 = fn(torch.zeros_like(g["x"]), qw, qlo, g["zeros"], g["scales"], bits, gs, bias=_t(b)).cpu().numpy()
    assert np.array_equal(y0.view(np.uint16), np.tile(b, (M, 1)).view(np.uint16))


@pytest.mark.parametrize("M,bits,gs", [(1, 4, -1), (16, 2, 32)])
def test_gemv_max_n(gpu, M, bits, gs):
    """The decode product at its largest N (2^20 columns: the largest grid, 16384 strips of
    64 columns; K = 64 is too short to split, so no workspace is used), compared with the
    oracle on sampled columns: the first and last 64 and 4000 drawn in between."""
    K, N = 64, 1 << 20
    _say(f"gemv max N M={M} K={K} N={N} bits={bits} gs={gs}")
    d = datagen.small_case(M, K, N, bits, gs, seed=M + bits)
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    y = gpu.qmm_gemv(g["x"], qw, qlo, g["zeros"], g["scales"], bits, gs).cpu().numpy()
    rng = np.random.default_rng(M)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N), rng.integers(0, N, 4000)]))
    y_ref, a = oracle.quantized_matmul_codes(d["x"], d["codes"][:, cols], d["zeros"][:, cols],
                                             d["scales"][:, cols], gs)
    _check(y[:, cols], y_ref, a, "gemv max N")


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("name", [n for n, wl in datagen.WORKLOADS.items() if wl.M <= 16])
def test_workload_gemv_full(gpu, name):
    wl = datagen.WORKLOADS[name]
    _say(f"workload {name} (full output)")
    d = datagen.generate(wl)
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], wl.bits)
    y = gpu.qmm_gemv(g["x"], qw, qlo, g["zeros"], g["scales"], wl.bits, wl.group_size).cpu().numpy()
    y_ref, a = oracle.quantized_matmul_codes(d["x"], d["codes"], d["zeros"], d["scales"], wl.group_size)
    _check(y, y_ref, a, name)
    # the prefill kernel computes the same function
    y2 = gpu.qmm_gemm(g["x"], qw, qlo, g["zeros"], g["scales"], wl.bits, wl.group_size).cpu().numpy()
    _check(y2, y_ref, a, name + " via gemm")


# Products wide enough for the 256 x 256 block tile, with partial tiles at the
# right and bottom edges, across code widths and group layouts: groups of whole
# 64-k slabs, groups of an odd number of 32-k units with a K tail, 32-k groups,
# one group per column with a K tail (with integer and with non-integer zero
# points). Sampled rows, every column, are compared with the oracle.
LARGE_TILE = [(4100, 512, 4104, 4, 128, False, False), (4100, 480, 4104, 4, 96, False, True),
              (4100, 512, 4104, 3, 64, False, False), (4100, 544, 4104, 8, -1, False, True),
              (4100, 544, 4104, 8, -1, True, False), (4100, 512, 4104, 2, 32, False, False),
              (4100, 512, 4104, 1, 64, False, False)]


@pytest.mark.parametrize("M,K,N,bits,gs,nonint,with_bias", LARGE_TILE)
def test_gemm_large_tile_sampled_rows(gpu, M, K, N, bits, gs, nonint, with_bias):
    _say(f"gemm large tile M={M} K={K} N={N} bits={bits} gs={gs} nonint-z={nonint} bias={with_bias}")
    d = datagen.small_case(M, K, N, bits, gs, seed=K + bits * 7 + (gs if gs > 0 else 3))
    if nonint:
        d["zeros"] = np.random.default_rng(5).uniform(-1.5, (1 << bits) + 0.5, size=d["zeros"].shape).astype(np.float16)
    b = np.random.default_rng(7).uniform(-4, 4, size=N).astype(np.float16) if with_bias else None
    g = _to_gpu_case(d)
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    y = gpu.qmm_gemm(g["x"], qw, qlo, g["zeros"], g["scales"], bits, gs, bias=None if b is None else _t(b))
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095, 4096, M - 2, M - 1], rng.choice(M, 40, replace=False)]))
    y_rows = y[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    w_ref = oracle.dequantize(d["codes"], d["scales"], d["zeros"], gs)
    y_ref, a = oracle.matmul(d["x"][rows], w_ref, b)
    _check(y_rows, y_ref, a, f"gemm large tile bits={bits} gs={gs}")


@pytest.mark.parametrize("M", [1, 16, 17, 300])
def test_functional_form(gpu, M):
    """quantized_matmul in the functional argument order: M <= 16 to the decode kernel, larger M to
    the prefill kernel, same function either way."""
    K, N, bits, gs = 512, 264, 4, 128
    _say(f"quantized_matmul M={M}")
    d = datagen.small_case(M, K, N, bits, gs, seed=M)
    qw_ref, qlo_ref = oracle.pack(d["codes"], bits)
    qw, qlo = _pack_gpu(gpu, d["codes"], bits)
    g = _to_gpu_case(d)
    y = gpu.quantized_matmul(g["x"], qw, g["zeros"], g["scales"], bits, gs, qweight_lo=qlo).cpu().numpy()
    y_ref, a = oracle.quantized_matmul(d["x"], qw_ref, qlo_ref, d["zeros"], d["scales"], bits, gs)
    _check(y, y_ref, a, f"quantized_matmul M={M}")


def test_workspace_shared_across_shapes(gpu):
    """Calls of different shapes share one cached workspace: wider problems place their
    partial sums where a narrower problem's would not, and the arrival counters never move."""
    cases = [(1, 1024, 4096, 4, 128), (1, 1024, 6144, 3, 128), (2, 2048, 264, 2, 64), (1, 1024, 4096, 4, 128),
             (1, 1024, 6144, 3, 128)]
    for i, (M, K, N, bits, gs) in enumerate(cases):
        _say(f"shared workspace call {i}: M={M} K={K} N={N} bits={bits} gs={gs}")
        y, y_ref, a = _run(gpu, "gemv", M, K, N, bits, gs, seed=i)
        _check(y, y_ref, a, f"shared workspace {i}")
