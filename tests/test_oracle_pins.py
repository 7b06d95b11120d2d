"""Pins of the CPU oracle to things other than itself.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
a fact fixed by the sources or by mathematics: hand-worked packed words and
products (tests/golden), exact rational and exact integer recomputation,
closed forms and invariants. ``test_planted_mistakes`` plants plausible bugs in
the oracle (on the CPU) and requires each to trip at least one check.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import datagen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _golden_codes(case):
    if isinstance(case["codes_k"], str):  # "k mod 8 for k = 0..31"
        return np.array([k % 8 for k in range(32)], dtype=np.uint8)
    return np.array(case["codes_k"], dtype=np.uint8)


# ---------------------------------------------------------------- packing pins

def check_pack_words_hand_worked():
    """Packed words of tests/golden/pack_words.json, in every column of a 3-column matrix."""
    for case in _load("pack_words.json")["cases"]:
        q = _golden_codes(case)
        codes = np.stack([q, q, q], axis=1)  # columns are independent
        bits = case["bits"]
        if bits == 3:
            p2, p1 = oracle.pack_3bit(codes)
            for col in range(3):
                assert p2[:, col].tolist() == case["plane2_words_int32"], case["name"]
                assert p1[:, col].tolist() == case["plane1_words_int32"], case["name"]
            assert np.array_equal(oracle.unpack_3bit(p2, p1, len(q)), codes), case["name"]
        else:
            w = oracle.pack_kmajor(codes, bits)
            assert w.dtype == np.int32
            for col in range(3):
                assert w[:, col].tolist() == case["words_int32"], case["name"]
            assert np.array_equal(oracle.unpack_kmajor(w, bits, len(q)), codes), case["name"]


def check_ascending_nibbles():
    """0x76543210 holds codes 0..7 in slot order at 4 bits, 0x10 / 0x32 / ... at 8 bits."""
    w = np.array([[0x76543210]], dtype=np.uint32).view(np.int32)
    assert oracle.unpack_kmajor(w, 4, 8)[:, 0].tolist() == list(range(8))
    assert oracle.unpack_kmajor(w, 8, 4)[:, 0].tolist() == [0x10, 0x32, 0x54, 0x76]
    # 2-bit slots of 0xE4 = 0b11100100 read 0,1,2,3 from the least significant end
    w2 = np.array([[0xE4E4E4E4]], dtype=np.uint32).view(np.int32)
    assert oracle.unpack_kmajor(w2, 2, 16)[:, 0].tolist() == [0, 1, 2, 3] * 4
    # 1-bit plane: bit k is code k
    w1 = np.array([[0x80000001]], dtype=np.uint32).view(np.int32)
    assert oracle.unpack_kmajor(w1, 1, 32)[:, 0].tolist() == [1] + [0] * 30 + [1]


def check_word_bijection(n_words=1 << 18, seed=7):
    """unpack then pack gives back every word, and pack then unpack every code matrix."""
    rng = np.random.default_rng(seed)
    for bits in oracle.PLANE_BITS:
        eps = 32 // bits
        words = rng.integers(0, 1 << 32, size=(n_words // 64, 64), dtype=np.uint64).astype(np.uint32)
        words[0, :4] = [0, 0xFFFFFFFF, 0x80000000, 0x7FFFFFFF]
        w = words.view(np.int32)
        q = oracle.unpack_kmajor(w, bits, w.shape[0] * eps)
        assert q.max() < (1 << bits)
        assert np.array_equal(oracle.pack_kmajor(q, bits), w), bits
        codes = rng.integers(0, 1 << bits, size=(eps * 6, 5), dtype=np.uint8)
        assert np.array_equal(oracle.unpack_kmajor(oracle.pack_kmajor(codes, bits), bits, eps * 6), codes), bits


def check_word_bijection_all_words_by_linearity(seed=11):
    """The round trip holds for all 2^32 words: unpack is a bit permutation.

    Unpacking moves word bit (k % eps) * bits + i to bit i of code k and does nothing else (shifts
    and masks), so it is linear over GF(2): checked on random pairs, unpack(a ^ b) equals
    unpack(a) ^ unpack(b). A linear map is fixed by its images of the 32 single-bit words; each
    image is one code with one bit set, at code b // bits, bit b % bits, and the 32 images are
    distinct, so unpack is a bijection of the 2^32 words onto the code arrays, and pack (checked to
    invert it on the same basis) is its inverse everywhere."""
    rng = np.random.default_rng(seed)
    for bits in oracle.PLANE_BITS:
        eps = 32 // bits
        seen = set()
        for b in range(32):
            w = np.array([[np.uint32(1) << np.uint32(b)]], dtype=np.uint32).view(np.int32)
            q = oracle.unpack_kmajor(w, bits, eps)[:, 0]
            nz = np.nonzero(q)[0]
            assert nz.tolist() == [b // bits], (bits, b, q.tolist())
            assert int(q[nz[0]]) == 1 << (b % bits), (bits, b)
            seen.add((int(nz[0]), int(q[nz[0]])))
            assert np.array_equal(oracle.pack_kmajor(q[:, None], bits), w), (bits, b)
        assert len(seen) == 32
        a = rng.integers(0, 1 << 32, size=(64, 16), dtype=np.uint64).astype(np.uint32)
        c = rng.integers(0, 1 << 32, size=(64, 16), dtype=np.uint64).astype(np.uint32)
        ua = oracle.unpack_kmajor(a.view(np.int32), bits, 64 * eps)
        uc = oracle.unpack_kmajor(c.view(np.int32), bits, 64 * eps)
        uac = oracle.unpack_kmajor((a ^ c).view(np.int32), bits, 64 * eps)
        assert np.array_equal(uac, ua ^ uc), bits


def check_out_of_range_codes_masked():
    """A code wider than the field is masked to its low bits and never spills into a neighbour."""
    codes = np.zeros((8, 1), dtype=np.uint8)
    codes[3, 0] = 0x1F  # 5 bits in a 4-bit field
    w = oracle.pack_kmajor(codes, 4)
    assert w.view(np.uint32)[0, 0] == 0xF << 12
    assert oracle.count_out_of_range(codes, 4) == 1
    codes3 = np.full((32, 1), 9, dtype=np.uint8)  # 0b1001 -> 0b001
    assert np.all(oracle.unpack_3bit(*oracle.pack_3bit(codes3), 32) == 1)


def check_three_bit_identity():
    """Every 3-bit value at every slot position of the 32-row plane period survives the two planes."""
    codes = np.array([[(k + c) % 8 for c in range(8)] for k in range(64)], dtype=np.uint8)
    p2, p1 = oracle.pack_3bit(codes)
    assert p2.shape == (4, 8) and p1.shape == (2, 8)
    hi = oracle.unpack_kmajor(p2, 2, 64).astype(int)
    lo = oracle.unpack_kmajor(p1, 1, 64).astype(int)
    assert np.array_equal((hi << 1) | lo, codes.astype(int))
    assert np.array_equal(hi, codes.astype(int) // 2) and np.array_equal(lo, codes.astype(int) % 2)


# ---------------------------------------------------------------- product pins

def check_dequant_examples_hand_worked():
    for case in _load("dequant_examples.json")["cases"]:
        codes = np.array(case["codes_kn"], dtype=np.uint8)
        s = np.array(case["scales_gn"], dtype=np.float16)
        z = np.array(case["zeros_gn"], dtype=np.float16)
        x = np.array(case["x"], dtype=np.float16)
        bias = np.array(case["bias_n"], dtype=np.float16) if "bias_n" in case else None
        for gs in case["group_sizes"]:
            w = oracle.dequantize(codes, s, z, gs)
            assert np.array_equal(w, np.array(case["w_kn"], dtype=np.float64)), case["name"]
            qw, qlo = oracle.pack(codes, case["bits"])
            y, a = oracle.quantized_matmul(x, qw, qlo, z, s, case["bits"], gs, bias=bias)
            assert np.array_equal(y, np.array(case["y"])), (case["name"], y)
            assert np.array_equal(a, np.array(case["a"])), (case["name"], a)


def check_dequant_fp16_hand_worked():
    """fp16 weights of tests/golden/dequant_examples.json 'fp16_cases', ties included."""
    for case in _load("dequant_examples.json")["fp16_cases"]:
        s = np.array([[int(case["scale_bits"], 16)]], dtype=np.uint16).view(np.float16)
        z = np.array([[case["zero"]]], dtype=np.float16)
        q = np.array([[case["q"]]], dtype=np.uint8)
        assert oracle.dequantize(q, s, z, -1)[0, 0] == case["exact"], case["name"]
        got = oracle.dequantize_fp16(q, s, z, -1).view(np.uint16)[0, 0]
        assert got == int(case["fp16_bits"], 16), (case["name"], hex(got))


def check_bf16_decode_every_pattern():
    """bf16_to_f64 agrees with the format's definition (sign, 8-bit exponent biased by 127, 7
    fraction bits, subnormals) on every finite bit pattern."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    finite = exp != 0xFF
    b = bits[finite]
    e = ((b >> 7) & 0xFF).astype(np.int64)
    f = (b & 0x7F).astype(np.float64)
    sign = np.where(b >> 15, -1.0, 1.0)
    want = np.where(e == 0, sign * f / 128.0 * 2.0 ** -126, sign * (1.0 + f / 128.0) * np.ldexp(1.0, e - 127))
    got = oracle.bf16_to_f64(b.astype(np.uint16))
    assert np.array_equal(got, want)


def check_bf16_encode_hand_worked():
    """f64_to_bf16 on the hand-worked values of tests/golden/dequant_examples.json, ties included."""
    d = _load("dequant_examples.json")
    for case in d["bf16_encode_cases"]:
        got = int(oracle.f64_to_bf16(np.array([case["value"]]))[0])
        assert got == int(case["bf16_bits"], 16), (case["name"], hex(got))
    for case in d["bf16_dequant_cases"]:
        s = np.array([[int(case["scale_bits"], 16)]], dtype=np.uint16)
        z = oracle.f64_to_bf16(np.array([[float(case["zero"])]]))
        q = np.array([[case["q"]]], dtype=np.uint8)
        assert oracle.dequantize(q, oracle.bf16_to_f64(s), oracle.bf16_to_f64(z), -1)[0, 0] == case["exact"]
        got = int(oracle.dequantize_bf16(q, s, z, -1)[0, 0])
        assert got == int(case["bf16_bits"], 16), (case["name"], hex(got))


def _round_half_even_bits(v: Fraction, frac_bits: int, emin: int) -> Fraction:
    """v rounded to frac_bits fraction bits (nearest, ties to even), exponents down to emin."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    v = abs(v)
    e = emin
    while v >= Fraction(2) ** (e + 1):
        e += 1
    step = Fraction(2) ** (e - frac_bits)
    n = v / step
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * step


def check_bf16_encode_against_exact_rounding(seed=12):
    """f64_to_bf16 equals exact rounding to 7 fraction bits on products of bf16 scales and codes,
    and on magnitudes below the bf16 normal range (fixed spacing 2^-133), ties among them."""
    rng = np.random.default_rng(seed)
    s = oracle.f64_to_bf16(rng.uniform(1e-4, 2.0, size=400))
    z = oracle.f64_to_bf16(rng.uniform(-3.0, 260.0, size=400))
    q = rng.integers(0, 256, size=400)
    v = oracle.bf16_to_f64(s) * (q - oracle.bf16_to_f64(z))
    # below 2^-126: random magnitudes in [2^-140, 2^-126), either sign, plus exact ties
    # (odd multiples of 2^-134, halfway between two representable values)
    tiny = np.ldexp(rng.uniform(1.0, 2.0, size=300), rng.integers(-140, -126, size=300))
    tiny *= np.where(rng.integers(0, 2, size=300) == 1, -1.0, 1.0)
    ties = np.ldexp(2.0 * rng.integers(0, 128, size=100) + 1.0, -134)
    v = np.concatenate([v, tiny, ties, -ties])
    got = oracle.bf16_to_f64(oracle.f64_to_bf16(v))
    for i in range(v.size):
        want = _round_half_even_bits(Fraction(float(v[i])), 7, -126)
        assert got[i] == float(want), (i, v[i], got[i], float(want))


def _round_half_even_fp16(v: Fraction) -> float:
    """The binary16 value nearest to v (ties to even), from the format's definition: 10 stored
    fraction bits, exponents -14..15, subnormals below 2^-14, overflow to infinity."""
    if v == 0:
        return 0.0
    sign = -1.0 if v < 0 else 1.0
    v = abs(v)
    e = -14
    while v >= Fraction(2) ** (e + 1) and e < 15:
        e += 1
    step = Fraction(2) ** (e - 10)
    n = v / step
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    out = fl * step
    if out > 65504:
        return sign * float("inf")
    return sign * float(out)


def check_dequant_fp16_against_exact_rounding(seed=11):
    """dequantize_fp16 equals the correctly rounded exact product, non-integer zero points included."""
    rng = np.random.default_rng(seed)
    for bits, gs in ((4, 32), (8, -1), (3, 32), (1, 32), (2, 64)):
        K, N = 64, 12
        codes = rng.integers(0, 1 << bits, size=(K, N)).astype(np.uint8)
        G = 1 if gs == -1 else K // gs
        s = rng.uniform(0.001, 0.3, size=(G, N)).astype(np.float16)
        z = rng.uniform(-2.0, (1 << bits) + 2.0, size=(G, N)).astype(np.float16)
        z[:, ::2] = np.round(z[:, ::2])
        w16 = oracle.dequantize_fp16(codes, s, z, gs)
        rows = K if gs == -1 else gs
        for k in range(0, K, 3):
            for n in range(N):
                g = k // rows
                exact = Fraction(float(s[g, n])) * (int(codes[k, n]) - Fraction(float(z[g, n])))
                assert float(w16[k, n]) == _round_half_even_fp16(exact), (bits, gs, k, n)


def _exact_y(x, codes, s, z, gs):
    """sum_k x[m,k] * s[g,n] * (q[k,n] - z[g,n]) in exact rationals, straight from the codes."""
    M, K = x.shape
    N = codes.shape[1]
    rows = K if gs == -1 else gs
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    xf = [[Fraction(float(v)) for v in row] for row in x]
    sf = [[Fraction(float(v)) for v in row] for row in s]
    zf = [[Fraction(float(v)) for v in row] for row in z]
    for m in range(M):
        for n in range(N):
            for k in range(K):
                g = k // rows
                t = xf[m][k] * sf[g][n] * (int(codes[k, n]) - zf[g][n])
                y[m][n] += t
                a[m][n] += abs(t)
    return y, a


def check_rational_brute_force(seed=3):
    """Tiny random products, including non-integer zero points, against exact rationals."""
    rng = np.random.default_rng(seed)
    for bits in (1, 2, 3, 4, 8):
        for K, gs in ((32, 32), (64, 16), (64, -1), (96, 32)):
            M, N = 2, 3
            codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)
            G = 1 if gs == -1 else K // gs
            s = rng.uniform(0.01, 0.5, size=(G, N)).astype(np.float16)
            z = rng.uniform(-2, (1 << bits) + 2, size=(G, N)).astype(np.float16)  # not integers
            x = rng.standard_normal((M, K)).astype(np.float16)
            qw, qlo = oracle.pack(codes, bits)
            y, a = oracle.quantized_matmul(x, qw, qlo, z, s, bits, gs)
            ye, ae = _exact_y(x, codes, s, z, gs)
            for m in range(M):
                for n in range(N):
                    tol = 1e-13 * float(ae[m][n]) + 1e-300
                    assert abs(y[m, n] - float(ye[m][n])) <= tol, (bits, K, gs, m, n)
                    assert abs(a[m, n] - float(ae[m][n])) <= tol, (bits, K, gs, m, n)


def check_matmul_is_the_triple_loop(seed=13):
    """numpy's float64 product against the sum written out as three loops (k ascending), on small
    products with and without a bias, and on the whole small decode workload (1 x 512 x 256)."""
    rng = np.random.default_rng(seed)
    for M, K, N in ((1, 32, 8), (3, 96, 5), (2, 256, 17)):
        x = rng.standard_normal((M, K)).astype(np.float16)
        w = rng.standard_normal((K, N))
        for bias in (None, rng.standard_normal(N).astype(np.float16)):
            y, a = oracle.matmul(x, w, bias)
            yl, al = oracle.matmul_triple_loop(x, w, bias)
            assert np.all(np.abs(y - yl) <= 1e-12 * al), (M, K, N)
            assert np.allclose(a, al, rtol=1e-12, atol=0)
    wl = datagen.WORKLOADS["gemv_m1_k512_n256_int4_g128"]
    d = datagen.generate(wl)
    qw, qlo = oracle.pack(d["codes"], wl.bits)
    y, a = oracle.quantized_matmul(d["x"], qw, qlo, d["zeros"], d["scales"], wl.bits, wl.group_size)
    yl, al = oracle.matmul_triple_loop(d["x"], oracle.dequantize(d["codes"], d["scales"], d["zeros"], wl.group_size))
    assert np.all(np.abs(y - yl) <= 1e-12 * al)


def check_exact_integer_recomputation(seed=11):
    """K = 4096 products with integer zero points, recomputed exactly in int64.

    fp16 values are integer multiples of 2**-24, so X = x * 2**24 is an int64;
    per group, S = sum_k X_k (q_k - z) is exact; y = 2**-24 * sum_g s_g S_g is
    summed as exact rationals.
    """
    for bits, gs in ((4, 128), (2, 64), (8, -1), (3, 128)):
        M, K, N = 2, 4096, 24
        d = datagen.small_case(M, K, N, bits, gs, seed=seed)
        codes, s, z, x = d["codes"], d["scales"], d["zeros"], d["x"]
        qw, qlo = oracle.pack(codes, bits)
        y, _ = oracle.quantized_matmul(x, qw, qlo, z, s, bits, gs)
        X = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
        assert np.array_equal(X.astype(np.float64) * 2.0 ** -24, x.astype(np.float64))
        rows = K if gs == -1 else gs
        zi = z.astype(np.int64)
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for g in range(K // rows):
                    seg = slice(g * rows, (g + 1) * rows)
                    S = int(np.dot(X[m, seg], codes[seg, n].astype(np.int64) - zi[g, n]))
                    tot += Fraction(float(s[g, n])) * S
                ye = float(tot / (1 << 24))
                assert abs(y[m, n] - ye) <= 1e-12 * max(1.0, abs(ye)), (bits, gs, m, n, y[m, n], ye)


def check_closed_form_constant_scale_zero(seed=5):
    """With one scale c and one zero d everywhere, y = c * (x @ Q - d * rowsum(x)), exact in int64."""
    rng = np.random.default_rng(seed)
    M, K, N = 3, 512, 40
    codes = rng.integers(0, 256, size=(K, N), dtype=np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float16)
    for gs in (128, -1):
        G = 1 if gs == -1 else K // gs
        s = np.full((G, N), 0.125, dtype=np.float16)
        z = np.full((G, N), 100, dtype=np.float16)
        y, _ = oracle.quantized_matmul_codes(x, codes, z, s, gs)
        X = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
        exact = 0.125 * (X @ codes.astype(np.int64) - 100 * X.sum(axis=1, keepdims=True)).astype(np.float64)
        assert np.allclose(y, exact * 2.0 ** -24, rtol=1e-12, atol=1e-12)
    # scale 1, zero 0: the plain product with the integer codes
    s1 = np.ones((1, N), dtype=np.float16)
    z0 = np.zeros((1, N), dtype=np.float16)
    y, a = oracle.quantized_matmul_codes(x, codes, z0, s1, -1)
    X = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    assert np.allclose(y, (X @ codes.astype(np.int64)) * 2.0 ** -24, rtol=1e-12, atol=1e-12)
    assert np.allclose(a, (np.abs(X) @ codes.astype(np.int64)) * 2.0 ** -24, rtol=1e-12, atol=1e-12)


def check_group_minus_one_is_single_group(seed=2):
    d = datagen.small_case(3, 256, 16, 4, -1, seed=seed)
    qw, _ = oracle.pack(d["codes"], 4)
    y1, a1 = oracle.quantized_matmul(d["x"], qw, None, d["zeros"], d["scales"], 4, -1)
    y2, a2 = oracle.quantized_matmul(d["x"], qw, None, d["zeros"], d["scales"], 4, 256)
    assert np.array_equal(y1, y2) and np.array_equal(a1, a2)
    assert oracle.num_groups(256, -1) == 1


def check_widths_agree_on_small_codes(seed=4):
    """Codes in [0, 7] packed as 3-bit planes, as 4-bit and as 8-bit give bit-identical products;
    codes in [0, 1] packed at every width (1-bit included) do too."""
    d = datagen.small_case(2, 256, 24, 3, 64, seed=seed)
    ys = []
    for bits in (3, 4, 8):
        qw, qlo = oracle.pack(d["codes"], bits)
        ys.append(oracle.quantized_matmul(d["x"], qw, qlo, d["zeros"], d["scales"], bits, 64)[0])
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
    d1 = datagen.small_case(2, 256, 24, 1, 64, seed=seed + 1)
    assert d1["codes"].max() <= 1
    ys = []
    for bits in (1, 2, 3, 4, 8):
        qw, qlo = oracle.pack(d1["codes"], bits)
        ys.append(oracle.quantized_matmul(d1["x"], qw, qlo, d1["zeros"], d1["scales"], bits, 64)[0])
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def check_bias_row(seed=5):
    """With x = 0 the product is the bias row exactly; otherwise y(bias) - bias == y (exact small values)."""
    d = datagen.small_case(3, 64, 16, 4, 32, seed=seed)
    qw, _ = oracle.pack(d["codes"], 4)
    b = np.linspace(-2, 2, 16).astype(np.float16)
    y0, a0 = oracle.quantized_matmul(np.zeros_like(d["x"]), qw, None, d["zeros"], d["scales"], 4, 32, bias=b)
    assert np.array_equal(y0, np.tile(b.astype(np.float64), (3, 1))) and np.array_equal(a0, np.abs(y0))
    y, a = oracle.quantized_matmul(d["x"], qw, None, d["zeros"], d["scales"], 4, 32)
    yb, ab = oracle.quantized_matmul(d["x"], qw, None, d["zeros"], d["scales"], 4, 32, bias=b)
    assert np.allclose(yb - b.astype(np.float64), y, rtol=0, atol=1e-12)
    assert np.allclose(ab - np.abs(b.astype(np.float64)), a, rtol=0, atol=1e-12)


def check_one_hot_rows(seed=9):
    """x = e_k selects row k of the dequantized weight: y[n] = s[g,n] * (q[k,n] - z[g,n]) exactly."""
    K, N, gs = 256, 8, 64
    d = datagen.small_case(1, K, N, 4, gs, seed=seed)
    qw, _ = oracle.pack(d["codes"], 4)
    for k in (0, 1, 7, 8, 63, 64, 127, 128, 200, 255):
        x = np.zeros((1, K), dtype=np.float16)
        x[0, k] = 1
        y, a = oracle.quantized_matmul(x, qw, None, d["zeros"], d["scales"], 4, gs)
        g = k // gs
        for n in range(N):
            want = Fraction(float(d["scales"][g, n])) * (int(d["codes"][k, n]) - Fraction(float(d["zeros"][g, n])))
            assert y[0, n] == float(want), (k, n)
            assert a[0, n] == abs(float(want))


def check_parity_rule():
    y_ref = np.array([[1.0, -2.0, 0.0]])
    a = np.array([[10.0, 4.0, 0.0]])
    bound = oracle.parity_bound(a)
    assert np.allclose(bound, [[0.021, 0.009, 0.001]])
    assert oracle.parity_report(y_ref + 0.99 * bound, y_ref, a)["ok"]
    assert not oracle.parity_report(y_ref + 1.01 * bound, y_ref, a)["ok"]
    bad = y_ref.copy()
    bad[0, 1] = np.nan
    r = oracle.parity_report(bad, y_ref, a)
    assert not r["ok"] and r["nonfinite"] == 1


def _two_roundings_worst(fmt):
    """Largest relative error of the kernels' rounding model on one term: the
    dequantized weight s * d rounded once to the format, its product with x
    (exact in float64, exact in fp32) rounded once to the format. Brute force
    over every significand of s and x in [1, 2) (every third one of s for fp16)
    and every integer code difference d in 1..255."""
    d = np.arange(1, 256, dtype=np.float64)
    if fmt == "bf16":
        sig = oracle.bf16_to_f64(np.arange(0x3F80, 0x4000, dtype=np.uint16))
        s_vals, x_vals = sig, sig

        def rnd(v):
            return oracle.bf16_to_f64(oracle.f64_to_bf16(v))
    else:
        sig = np.arange(0x3C00, 0x4000, dtype=np.uint16).view(np.float16).astype(np.float64)
        s_vals, x_vals = sig[::3], sig

        def rnd(v):
            return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)
    worst = 0.0
    for s in s_vals:
        w = s * d                      # exact
        wq = rnd(w)
        exact = x_vals[:, None] * w[None, :]
        y = rnd(x_vals[:, None] * wq[None, :])
        worst = max(worst, float(np.max(np.abs(y - exact) / exact)))
    return worst


def check_tolerance_covers_the_rounding_model():
    """REL_TOL (fp16) and REL_TOL_BF16 must cover two roundings to the format
    (weight and output) plus fp32 accumulation over up to K = 16384 terms
    (K * 2^-24). A format with p significant bits rounds with relative error up
    to 2^-p: 2^-11 for fp16, 2^-8 for bf16 (7 stored fraction bits plus the
    implicit one)."""
    acc = 16384 * 2.0 ** -24
    for fmt, tol, p in (("fp16", oracle.REL_TOL, 11), ("bf16", oracle.REL_TOL_BF16, 8)):
        worst = _two_roundings_worst(fmt)
        u = 2.0 ** -p
        assert worst <= 2 * u + u * u, (fmt, worst)   # the model's own bound
        assert worst + acc <= tol, (fmt, worst, tol)
    # the brute force reaches the bf16 worst case: both roundings at close to 2^-8
    assert _two_roundings_worst("bf16") > 1.9 * 2.0 ** -8


# ---------------------------------------------------------------- strip-major storage order

def check_strips_hand_worked():
    # A (2, 24) plane with word (r, n) = 100 r + n, laid out by hand: strip 0
    # holds columns 0-15 of row 0, then of row 1; strip 1 holds columns 16-23
    # of each row followed by 8 zero words of padding.
    words = np.array([[100 * r + n for n in range(24)] for r in range(2)], dtype=np.int32)
    want = np.array([
        [[0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15],
         [100, 101, 102, 103, 104, 105, 106, 107, 108, 109, 110, 111, 112, 113, 114, 115]],
        [[16, 17, 18, 19, 20, 21, 22, 23, 0, 0, 0, 0, 0, 0, 0, 0],
         [116, 117, 118, 119, 120, 121, 122, 123, 0, 0, 0, 0, 0, 0, 0, 0]],
    ], dtype=np.int32)
    got = oracle.to_strips(words)
    assert got.shape == (2, 2, 16) and np.array_equal(got, want)
    # flat index of word (r, n): ((n // 16) * rows + r) * 16 + n % 16
    flat = got.reshape(-1)
    assert flat[(1 * 2 + 1) * 16 + 5] == 121 and flat[(0 * 2 + 1) * 16 + 15] == 115
    assert np.array_equal(oracle.from_strips(want, 24), words)


def check_strips_round_trip_and_padding():
    rng = np.random.default_rng(5)
    for rows, N in ((1, 8), (3, 16), (5, 40), (64, 136)):
        w = rng.integers(-2**31, 2**31, size=(rows, N), dtype=np.int64).astype(np.int32)
        t = oracle.to_strips(w)
        assert t.shape == ((N + 15) // 16, rows, 16)
        assert np.array_equal(oracle.from_strips(t, N), w)
        # a permutation of the words plus zero padding: the multisets agree
        pad = t.size - w.size
        assert np.array_equal(np.sort(t.reshape(-1)), np.sort(np.concatenate([w.reshape(-1), np.zeros(pad, np.int32)])))
        # each strip of the output is contiguous: its rows are the plane's 16 columns
        for s_ in range(t.shape[0]):
            cols = slice(16 * s_, min(16 * s_ + 16, N))
            assert np.array_equal(t[s_, :, : cols.stop - cols.start], w[:, cols])


CHECKS = [
    check_strips_hand_worked, check_strips_round_trip_and_padding,
    check_pack_words_hand_worked, check_ascending_nibbles, check_word_bijection,
    check_word_bijection_all_words_by_linearity,
    check_out_of_range_codes_masked, check_three_bit_identity, check_dequant_examples_hand_worked,
    check_dequant_fp16_hand_worked, check_dequant_fp16_against_exact_rounding, check_bias_row,
    check_bf16_decode_every_pattern, check_bf16_encode_hand_worked, check_bf16_encode_against_exact_rounding,
    check_rational_brute_force, check_matmul_is_the_triple_loop, check_exact_integer_recomputation,
    check_closed_form_constant_scale_zero,
    check_group_minus_one_is_single_group, check_widths_agree_on_small_codes, check_one_hot_rows,
    check_parity_rule, check_tolerance_covers_the_rounding_model,
]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(check):
    check()


# ---------------------------------------------------------------- planted mistakes

def _mut_pack_slot_reversed(codes, bits):
    K, N = codes.shape
    eps = 32 // bits
    words = np.zeros((K // eps, N), dtype=np.uint32)
    for k in range(K):
        words[k // eps] |= (codes[k].astype(np.uint32) & np.uint32((1 << bits) - 1)) << np.uint32((eps - 1 - k % eps) * bits)
    return words.view(np.int32)


def _mut_unpack_arith_shift(words, bits, K):
    s = np.asarray(words).astype(np.int64)  # sign-extending, no mask on the top slot
    eps = 32 // bits
    q = np.empty((K, s.shape[1]), dtype=np.int64)
    for k in range(K):
        q[k] = s[k // eps] >> ((k % eps) * bits)
        if k % eps != eps - 1:
            q[k] &= (1 << bits) - 1
    return q.astype(np.int64)


def _mut_dequant_no_zero(q, scales, zeros, group_size):
    K = q.shape[0]
    rows = K if group_size == -1 else group_size
    g = np.arange(K) // rows
    return scales.astype(np.float64)[g] * q.astype(np.float64)


def _mut_dequant_wrong_group(q, scales, zeros, group_size):
    K = q.shape[0]
    rows = K if group_size == -1 else group_size
    g = (np.arange(K) // rows + 1) % (K // rows)  # off by one group
    return scales.astype(np.float64)[g] * (q.astype(np.float64) - zeros.astype(np.float64)[g])


def _mut_dequant_sign(q, scales, zeros, group_size):
    K = q.shape[0]
    rows = K if group_size == -1 else group_size
    g = np.arange(K) // rows
    return scales.astype(np.float64)[g] * (zeros.astype(np.float64)[g] - q.astype(np.float64))


def _mut_matmul_transposed_x(x, w, bias=None):
    x64 = np.asarray(x).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    xr = x64[:, ::-1]  # k index reversed
    y, a = xr @ w64, np.abs(xr) @ np.abs(w64)
    if bias is not None:
        b = np.asarray(bias).astype(np.float64).reshape(1, -1)
        y, a = y + b, a + np.abs(b)
    return y, a


def _mut_3bit_planes_swapped(codes):
    q = np.asarray(codes).astype(np.uint8) & 7
    return oracle.pack_kmajor(q & 1, 2), oracle.pack_kmajor(q >> 1, 1)


def _mut_matmul_drops_bias(x, w, bias=None):
    x64 = np.asarray(x).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    return x64 @ w64, np.abs(x64) @ np.abs(w64)


def _mut_fp16_truncates(q, scales, zeros, group_size):
    w = oracle.dequantize(q, scales, zeros, group_size)
    t = w.astype(np.float16)
    # round toward zero instead of to nearest
    over = np.abs(t.astype(np.float64)) > np.abs(w)
    t[over] = np.nextafter(t[over], np.float16(0))
    return t


def _mut_bf16_truncates(v):
    d = np.asarray(v, dtype=np.float64)
    return (d.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _mut_bf16_subnormal_truncates(v):
    # correct in the normal range, truncating below 2^-126
    d = np.asarray(v, dtype=np.float64)
    u = d.view(np.uint64)
    low = u & np.uint64((1 << 45) - 1)
    q = u >> np.uint64(45)
    half = np.uint64(1 << 44)
    q = q + ((low > half) | ((low == half) & ((q & np.uint64(1)) == np.uint64(1)))).astype(np.uint64)
    r = (q << np.uint64(45)).view(np.float64)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _mut_strips_rows_major(words):
    rows, N = words.shape  # strips ordered column-major inside a strip
    out = np.zeros(((N + 15) // 16, 16, rows), dtype=words.dtype)
    for n in range(N):
        out[n // 16, n % 16, :] = words[:, n]
    return out.reshape((N + 15) // 16, rows, 16)


def _mut_strips_width_8(words):
    rows, N = words.shape
    out = np.zeros(((N + 15) // 16, rows, 16), dtype=words.dtype)
    flat = out.reshape(-1)
    for r in range(rows):
        for n in range(N):
            flat[((n // 8) * rows + r) * 8 + n % 8] = words[r, n]
    return out


MUTATIONS = {
    "strips_rows_major": ("to_strips", _mut_strips_rows_major),
    "strips_width_8": ("to_strips", _mut_strips_width_8),
    "pack_slot_reversed": ("pack_kmajor", _mut_pack_slot_reversed),
    "unpack_arith_shift": ("unpack_kmajor", _mut_unpack_arith_shift),
    "dequant_no_zero": ("dequantize", _mut_dequant_no_zero),
    "dequant_wrong_group": ("dequantize", _mut_dequant_wrong_group),
    "dequant_sign": ("dequantize", _mut_dequant_sign),
    "matmul_reversed_k": ("matmul", _mut_matmul_transposed_x),
    "three_bit_planes_swapped": ("pack_3bit", _mut_3bit_planes_swapped),
    "matmul_drops_bias": ("matmul", _mut_matmul_drops_bias),
    "fp16_truncates": ("dequantize_fp16", _mut_fp16_truncates),
    "bf16_truncates": ("f64_to_bf16", _mut_bf16_truncates),
    "bf16_subnormal_truncates": ("f64_to_bf16", _mut_bf16_subnormal_truncates),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(name, monkeypatch):
    """Each plausible bug planted in the oracle makes at least one pin fail."""
    from oracle import qmm_oracle
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(qmm_oracle, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for check in CHECKS:
        if check is check_word_bijection:
            continue  # the slow one adds nothing the others miss here
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"planted mistake {name} was not caught by any pin"
