"""The 16-column strip-major weight layout on the GPU.

* qmm_to_strips against the oracle's definition of the order, word for word,
  on ragged widths (N % 16 == 8) and row counts that are not powers of two;
  qmm_from_strips gives the K-major plane back.
* The products with QMM_STRIPS read the same words at other addresses and
  run the same arithmetic in the same order, so their results must equal the
  K-major calls bit for bit. That is checked for every compiled variant of
  the wave-local decode kernel (the smallest shape of each), for split-K
  decode plans, for every GEMM tile shape (ragged N, a K tail) and every
  code width, in fp16 and bf16. Every fourth decode variant and each GEMM
  case is also compared with the oracle on sampled columns, and the
  4096 x 4096 4-bit decode workload on all outputs.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import gemv_plan_cases as cases
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


def _tb(u):  # bf16 bit patterns (uint16) -> a bf16 tensor
    return torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).to(DEV)


def _to_strips(gpu, qw, qlo):
    return gpu.qmm_to_strips(qw), None if qlo is None else gpu.qmm_to_strips(qlo)


@pytest.mark.parametrize("rows,N", [(1, 8), (3, 24), (5, 16), (64, 4096), (257, 4104), (16, 65544)])
def test_to_strips_is_the_defined_order(gpu, rows, N):
    _say(f"to_strips rows={rows} N={N}")
    rng = np.random.default_rng(rows * 7 + N)
    w = rng.integers(-2**31, 2**31, size=(rows, N), dtype=np.int64).astype(np.int32)
    got = gpu.qmm_to_strips(_t(w))
    torch.cuda.synchronize()
    want = oracle.to_strips(w)
    assert tuple(got.shape) == want.shape
    assert np.array_equal(got.cpu().numpy(), want)
    back = gpu.qmm_from_strips(got, N)
    assert np.array_equal(back.cpu().numpy(), w)


def _gemv_pair(gpu, x, qw, qlo, z, s, bits, gs, bias, sw, slo):
    y0 = gpu.qmm_gemv(x, qw, qlo, z, s, bits, gs, bias=bias)
    y1 = gpu.qmm_gemv(x, sw, slo, z, s, bits, gs, bias=bias, strips=True)
    return y0, y1


def _bits_of(y):
    return y.view(torch.int16).cpu().numpy()


CASES = cases.wave_cases()
KEYS = list(CASES)
SPLIT = [(1, 4096, 1024, 4, 128), (4, 8192, 512, 8, -1), (8, 4096, 8200, 3, 128), (16, 4096, 12288, 8, -1),
         (3, 8192, 136, 2, 64), (1, 2048, 1032, 1, -1)]


def _decode_case(gpu, M, K, N, bits, gs, seed, dt, check_oracle):
    G = oracle.num_groups(K, gs)
    codes = datagen.draw_codes(K, N, bits, seed=seed)
    qw, qlo = gpu.qmm_pack(_t(codes), bits)
    sw, slo = _to_strips(gpu, qw, qlo)
    x32 = datagen.draw_x_f32(M, K, seed)
    s32 = datagen.draw_scales_f32(G, N, 0.005, 0.05, seed)
    z64 = np.random.default_rng(seed).integers(0, 1 << bits, size=(G, N)).astype(np.float64)
    if seed % 3 == 0:  # some non-integer zero points: the remainder pass runs too
        z64[:, ::5] += 0.37
    b32 = np.random.default_rng(seed + 1).uniform(-4, 4, size=N).astype(np.float32) if seed % 2 else None
    if dt == "fp16":
        x, s, z = x32.astype(np.float16), s32.astype(np.float16), z64.astype(np.float16)
        b = None if b32 is None else b32.astype(np.float16)
        y0, y1 = _gemv_pair(gpu, _t(x), qw, qlo, _t(z), _t(s), bits, gs, None if b is None else _t(b), sw, slo)
        xr, sr, zr, br = x, s, z, b
        tol = oracle.REL_TOL
    else:
        xb, sb, zb = datagen.round_to_bf16(x32), datagen.round_to_bf16(s32), datagen.round_to_bf16(z64.astype(np.float32))
        bb = None if b32 is None else datagen.round_to_bf16(b32)
        y0, y1 = _gemv_pair(gpu, _tb(xb), qw, qlo, _tb(zb), _tb(sb), bits, gs, None if bb is None else _tb(bb), sw, slo)
        f = oracle.bf16_to_f64
        xr, sr, zr, br = f(xb), f(sb), f(zb), None if bb is None else f(bb)
        tol = oracle.REL_TOL_BF16
    a0, a1 = _bits_of(y0), _bits_of(y1)
    assert np.array_equal(a0, a1), (M, K, N, bits, gs, dt, int((a0 != a1).sum()))
    if check_oracle:
        cols = np.unique(np.r_[np.arange(min(16, N)), np.arange(16, N, 37), np.arange(max(0, N - 16), N)])
        y_ref, a = oracle.quantized_matmul_codes(xr, codes[:, cols], zr[:, cols], sr[:, cols], gs,
                                                 bias=None if br is None else br[cols])
        if dt == "fp16":
            got = y1.cpu().numpy()[:, cols].astype(np.float64)
        else:
            got = oracle.bf16_to_f64(a1.view(np.uint16)[:, cols])
        rep = oracle.parity_report(got, y_ref, a, rel_tol=tol)
        _say(f"    oracle: max|err|/bound={rep['max_ratio']:.4f} violations={rep['violations']}")
        assert rep["ok"] and rep["max_ratio"] < 0.35, rep


@pytest.mark.parametrize("key", KEYS, ids=["b{}_v{}_w{}_u{}_g{}".format(*k) for k in KEYS])
def test_gemv_strips_equals_k_major_wave_variants(gpu, key):
    K, N, gs, ms = CASES[key]
    idx = KEYS.index(key)
    for r, M in enumerate((ms[0], ms[-1]) if len(ms) > 1 else ms):
        dt = ("fp16", "bf16")[(idx + r) % 2]
        _say(f"strips gemv {key}: M={M} K={K} N={N} gs={gs} {dt}")
        _decode_case(gpu, M, K, N, key[0], gs, 500 + 3 * idx + r, dt, check_oracle=(idx % 4 == 0 and r == 0))


@pytest.mark.parametrize("M,K,N,bits,gs", SPLIT, ids=[f"m{c[0]}_k{c[1]}_n{c[2]}_b{c[3]}_g{c[4]}" for c in SPLIT])
def test_gemv_strips_equals_k_major_split_plans(gpu, M, K, N, bits, gs):
    p = gpu.gemv_plan_info(M, K, N, bits, gs)
    assert p["kernel"] == 0 and p["ksplit"] > 1, p
    for i, dt in enumerate(("fp16", "bf16")):
        _say(f"strips gemv split M={M} K={K} N={N} bits={bits} gs={gs} {dt} plan {p}")
        _decode_case(gpu, M, K, N, bits, gs, 900 + M + bits + 7 * i, dt, check_oracle=True)


# (M, K, N, group_size): the 256 x 256, 128 x 128 and both 64 x 64 tile shapes;
# ragged N (N % 16 == 8, so the last strip is padded) and a K tail (K % 64 != 0).
GEMM = [(2048, 256, 8200, 128), (1024, 256, 4104, -1), (96, 2048, 1032, 128), (300, 96, 136, 32)]


@pytest.mark.parametrize("bits", (1, 2, 3, 4, 8))
@pytest.mark.parametrize("M,K,N,gs", GEMM, ids=[f"m{c[0]}_k{c[1]}_n{c[2]}_g{c[3]}" for c in GEMM])
def test_gemm_strips_equals_k_major(gpu, M, K, N, gs, bits):
    p = gpu.gemm_plan_info(M, K, N, bits, gs)
    seed = M + K + N + bits
    d = datagen.small_case(M, K, N, bits, gs, seed=seed)
    codes = d["codes"]
    qw, qlo = gpu.qmm_pack(_t(codes), bits)
    sw, slo = _to_strips(gpu, qw, qlo)
    for i, dt in enumerate(("fp16", "bf16")):
        _say(f"strips gemm M={M} K={K} N={N} bits={bits} gs={gs} {dt} tile {p['bm']}x{p['bn']} kg={p['kgroups']}")
        if dt == "fp16":
            x, z, s = _t(d["x"]), _t(d["zeros"]), _t(d["scales"])
        else:
            x = _tb(datagen.round_to_bf16(d["x"].astype(np.float32)))
            z = _tb(datagen.round_to_bf16(d["zeros"].astype(np.float32)))
            s = _tb(datagen.round_to_bf16(d["scales"].astype(np.float32)))
        y0 = gpu.qmm_gemm(x, qw, qlo, z, s, bits, gs)
        y1 = gpu.qmm_gemm(x, sw, slo, z, s, bits, gs, strips=True)
        a0, a1 = _bits_of(y0), _bits_of(y1)
        assert np.array_equal(a0, a1), (dt, int((a0 != a1).sum()))
        if dt == "fp16":
            rows = np.unique(np.r_[0, M // 2, M - 1])
            cols = np.unique(np.r_[np.arange(0, N, 29), N - 1])
            y_ref, a = oracle.quantized_matmul_codes(d["x"][rows], codes[:, cols], d["zeros"][:, cols],
                                                     d["scales"][:, cols], gs)
            rep = oracle.parity_report(y1.cpu().numpy()[rows][:, cols].astype(np.float64), y_ref, a)
            _say(f"    oracle: max|err|/bound={rep['max_ratio']:.4f} violations={rep['violations']}")
            assert rep["ok"] and rep["max_ratio"] < 0.35, rep


def test_headline_decode_workload_in_strips(gpu):
    wl = datagen.WORKLOADS["gemv_m1_k4096_n4096_int4_g128"]
    _say(f"strips: {wl.name}")
    d = datagen.generate(wl)
    qw, qlo = gpu.qmm_pack(_t(d["codes"]), wl.bits)
    sw, _ = _to_strips(gpu, qw, qlo)
    x, z, s = _t(d["x"]), _t(d["zeros"]), _t(d["scales"])
    y0 = gpu.qmm_gemv(x, qw, qlo, z, s, wl.bits, wl.group_size)
    y1 = gpu.qmm_gemv(x, sw, None, z, s, wl.bits, wl.group_size, strips=True)
    assert np.array_equal(_bits_of(y0), _bits_of(y1))
    y_ref, a = oracle.quantized_matmul_codes(d["x"], d["codes"], d["zeros"], d["scales"], wl.group_size)
    rep = oracle.parity_report(y1.cpu().numpy().astype(np.float64), y_ref, a)
    _say(f"    oracle, all {y_ref.size} outputs: max|err|/bound={rep['max_ratio']:.4f}")
    assert rep["ok"] and rep["max_ratio"] < 0.35, rep


def test_strips_shape_checks(gpu):
    codes = datagen.draw_codes(256, 64, 4, seed=3)
    qw, _ = gpu.qmm_pack(_t(codes), 4)
    sw = gpu.qmm_to_strips(qw)
    x = torch.zeros((1, 256), dtype=torch.float16, device=DEV)
    z = torch.zeros((2, 64), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):  # K-major words passed as strips
        gpu.qmm_gemv(x, qw, None, z, z, 4, 128, strips=True)
    with pytest.raises(ValueError):  # strips of another width
        gpu.qmm_gemv(x, sw[:, :16], None, z, z, 4, 128, strips=True)
    with pytest.raises(ValueError):
        gpu.qmm_from_strips(sw, 80)
