"""CPU oracle for the weight-only, group-wise asymmetric integer quantized matmul.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP
library and its Python binding) never calls it, and it shares no code with
that path.

What it computes, step by step, in the order the sources state it:

* Packing: integer codes are stored K-major in 32-bit words, ``eps = 32 // bits``
  codes per word; code ``k`` of column ``n`` sits in word ``k // eps`` of that
  column at bit offset ``(k % eps) * bits``. (dashq_kernel.py, module
  docstring and ``_pack_kmajor`` / ``_unpack_kmajor``.)
* 3-bit codes are two planes: a 2-bit plane holding ``q >> 1`` and a 1-bit
  plane holding ``q & 1``; ``q = (hi << 1) | lo``. (dashq_kernel.py, module
  docstring, ``TritonQuantLinear.__init__`` and ``dequantize_weight``.) Widths
  1, 2, 3, 4 and 8 are supported (dashq_kernel.py, ``SUPPORTED_NBITS``).
* Groups: row ``k`` of the weight belongs to group ``k // group_size``;
  ``group_size == -1`` means one group for the whole column.
  (GPTQModel-Compatible Triton Kernel README, "Group Quantization".)
* Dequantization: ``w[k, n] = scale[g, n] * (q[k, n] - zero[g, n])``.
  (GPTQModel-Compatible Triton Kernel README, "Dequantization Formula";
  dashq_kernel.py, ``dequantize_weight``.)
* Product: ``y = x @ w`` with x of shape (M, K). (GPTQModel-Compatible Triton
  Kernel README, "API Reference", ``gptqmodel_quantized_matmul``.) ``matmul``
  takes numpy's float64 product (a library primitive, for the sizes of the
  workloads); ``matmul_triple_loop`` is the same sum written out as three
  loops, and the pins hold the two together on small products. An optional
  bias row is added to every row of y (dashq_kernel.py, ``TritonQuantLinear``:
  the accumulator starts from the bias).
* The dequantized weight as fp16 (dashq_kernel.py, ``dequantize_weight``): the
  exact product rounded once to the nearest half, ties to even.
* bf16 activations, scales, zero points and output (dashq_kernel.py: the module
  keeps scales and zeros in its output dtype and returns the product in the
  activations' dtype). bf16 values travel as uint16 bit patterns (numpy has no
  bf16 type); they are decoded exactly and the same float64 reference applies.
  The bf16 tolerance is re-derived from the format: bf16 keeps 8 significant
  bits, so one rounding to nearest errs by up to 2^-8 relative. One rounding
  of each dequantized weight (2^-8), the output rounding (2^-8) and fp32
  accumulation (K 2^-24) stay below 9e-3 * sum_k |x_k w_kn| up to K = 16384,
  as the fp16 rule's 2e-3 covers 2 * 2^-11 + K 2^-24.

Arithmetic is float64 throughout. Every fp16 input is widened to float64
exactly; for the workloads' integer zero points every product ``x * w`` is exact
in float64, so the only rounding is in the K-term sums (relative error about
K * 2**-53). The matrix product uses numpy's float64 matmul as a library step.

* The 16-column strip-major order of a word plane (a storage order of the
  library, not of the pages: the same words, reordered once at load time so
  that each 16-column strip is contiguous): word ``(r, n)`` of a (rows, N)
  plane goes to ``[n // 16, r, n % 16]`` of a (ceil(N / 16), rows, 16) array,
  the last strip's columns past N zero. ``to_strips`` / ``from_strips`` write
  that definition out element by element.

Parity pins: every function here is pinned by CPU tests (hand-worked words and
products from the definitions, exact integer and rational recomputation,
invariants).
"""
from __future__ import annotations

import numpy as np

# Bit widths whose codes pack into one plane of 32-bit words. 3 is handled as
# two planes (2 + 1); 1 is the width of the low 3-bit plane.
PLANE_BITS = (1, 2, 4, 8)
SUPPORTED_BITS = (1, 2, 3, 4, 8)

# Element-wise parity rule: |y - y_ref| <= REL_TOL * sum_k |x_k w_kn| + ABS_TOL.
REL_TOL = 2e-3
ABS_TOL = 1e-3
# The same rule for bf16 data (see the module docstring for the derivation).
REL_TOL_BF16 = 9e-3


def elements_per_word(bits: int) -> int:
    """Codes per 32-bit word for a single plane of ``bits``-bit codes."""
    if bits not in PLANE_BITS:
        raise ValueError(f"no single-plane packing for {bits}-bit codes")
    return 32 // bits


def count_out_of_range(codes: np.ndarray, bits: int) -> int:
    """Number of codes that do not fit in ``bits`` bits (they are masked on packing)."""
    return int(np.count_nonzero(np.asarray(codes, dtype=np.int64) >> bits))


def pack_kmajor(codes: np.ndarray, bits: int) -> np.ndarray:
    """(K, N) codes -> (K // eps, N) int32 words, K-major.

    Code k of a column goes to word k // eps of that column, at bit offset
    (k % eps) * bits; codes are first masked to ``bits`` bits.
    """
    codes = np.asarray(codes)
    K, N = codes.shape
    eps = elements_per_word(bits)
    if K % eps:
        raise ValueError(f"K={K} is not a multiple of {eps} codes per word")
    mask = np.uint32((1 << bits) - 1)
    words = np.zeros((K // eps, N), dtype=np.uint32)
    for k in range(K):
        shift = np.uint32((k % eps) * bits)
        words[k // eps] |= (codes[k].astype(np.uint32) & mask) << shift
    return words.view(np.int32)


def unpack_kmajor(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    """(K // eps, N) int32 words -> (K, N) uint8 codes; inverse of ``pack_kmajor``.

    Words are read as unsigned 32-bit patterns, so shifts are logical.
    """
    u = np.asarray(words).view(np.uint32)
    eps = elements_per_word(bits)
    if u.shape[0] * eps < K:
        raise ValueError("too few word rows for K")
    mask = np.uint32((1 << bits) - 1)
    q = np.empty((K, u.shape[1]), dtype=np.uint8)
    for k in range(K):
        shift = np.uint32((k % eps) * bits)
        q[k] = (u[k // eps] >> shift) & mask
    return q


def pack_3bit(codes: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(K, N) codes in [0, 7] -> (2-bit plane (K/16, N), 1-bit plane (K/32, N)).

    The 2-bit plane holds the top two bits of each code, the 1-bit plane the
    lowest bit. Codes are masked to 3 bits first.
    """
    q = np.asarray(codes).astype(np.uint8) & np.uint8(7)
    return pack_kmajor(q >> 1, 2), pack_kmajor(q & 1, 1)


def unpack_3bit(plane2: np.ndarray, plane1: np.ndarray, K: int) -> np.ndarray:
    """Two planes -> (K, N) codes, q = (hi << 1) | lo."""
    hi = unpack_kmajor(plane2, 2, K).astype(np.uint8)
    lo = unpack_kmajor(plane1, 1, K).astype(np.uint8)
    return (hi << 1) | lo


def pack(codes: np.ndarray, bits: int) -> tuple[np.ndarray, np.ndarray | None]:
    """Pack for any supported width: (qweight, qweight_lo); qweight_lo is None unless bits == 3."""
    if bits == 3:
        return pack_3bit(codes)
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"unsupported bit width {bits}")
    return pack_kmajor(codes, bits), None


def unpack(qweight: np.ndarray, qweight_lo: np.ndarray | None, bits: int, K: int) -> np.ndarray:
    if bits == 3:
        return unpack_3bit(qweight, qweight_lo, K)
    if bits not in SUPPORTED_BITS:
        raise ValueError(f"unsupported bit width {bits}")
    return unpack_kmajor(qweight, bits, K)


def group_rows(K: int, group_size: int) -> int:
    """Rows of the weight per group: group_size, or K when group_size == -1."""
    if group_size == -1:
        return K
    if group_size <= 0 or K % group_size:
        raise ValueError(f"group_size={group_size} does not divide K={K}")
    return group_size


def num_groups(K: int, group_size: int) -> int:
    return K // group_rows(K, group_size)


def dequantize(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group_size: int) -> np.ndarray:
    """(K, N) codes -> (K, N) float64 weights, w = scale[g] * (q - zero[g]), g = k // group_size."""
    q = np.asarray(q)
    K = q.shape[0]
    rows = group_rows(K, group_size)
    g = np.arange(K) // rows
    s = np.asarray(scales).astype(np.float64)
    z = np.asarray(zeros).astype(np.float64)
    if s.shape[0] != K // rows or z.shape[0] != K // rows:
        raise ValueError("scales/zeros must have one row per group")
    return s[g] * (q.astype(np.float64) - z[g])


def dequantize_fp16(q: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group_size: int) -> np.ndarray:
    """(K, N) codes -> (K, N) fp16 weights: the float64 product rounded once to fp16 (nearest, ties to even).

    With fp16 scales and zero points and codes below 256 the float64 product is
    exact, so this is the correctly rounded fp16 value of s * (q - z).
    """
    return dequantize(q, scales, zeros, group_size).astype(np.float16)


def matmul(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """y = x @ w (+ bias) and the tolerance reference a = sum_k |x_k * w_kn| (+ |bias|), both float64."""
    x64 = np.asarray(x).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    y, a = x64 @ w64, np.abs(x64) @ np.abs(w64)
    if bias is not None:
        b = np.asarray(bias).astype(np.float64).reshape(1, -1)
        y, a = y + b, a + np.abs(b)
    return y, a


def matmul_triple_loop(x: np.ndarray, w: np.ndarray, bias: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """The product written out as the definition reads: for every (m, n), the sum over k of
    x[m, k] * w[k, n] in float64, k ascending (bias first when given), and the tolerance reference
    a alongside. Plain Python loops, for small cases (the pins hold ``matmul`` to it)."""
    x64 = np.asarray(x).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float64)
    M, K = x64.shape
    N = w64.shape[1]
    b = None if bias is None else np.asarray(bias).astype(np.float64).reshape(-1)
    y = np.zeros((M, N), dtype=np.float64)
    a = np.zeros((M, N), dtype=np.float64)
    xl, wl = x64.tolist(), w64.tolist()
    for m in range(M):
        for n in range(N):
            acc = 0.0 if b is None else float(b[n])
            aa = 0.0 if b is None else abs(float(b[n]))
            for k in range(K):
                t = xl[m][k] * wl[k][n]
                acc += t
                aa += abs(t)
            y[m, n], a[m, n] = acc, aa
    return y, a


def quantized_matmul(x, qweight, qweight_lo, zeros, scales, bits: int, group_size: int, bias=None):
    """Reference for ``y = x @ dequantize(qweight) (+ bias)`` from packed words.

    Arguments follow the functional statement of the problem (x, packed weight,
    zeros, scales, bits, group_size); ``qweight_lo`` is the 1-bit plane for
    3-bit weights; ``bias`` is an optional (N,) row. Returns (y, a) in float64,
    a being the tolerance reference.
    """
    K = np.asarray(x).shape[1]
    q = unpack(qweight, qweight_lo, bits, K)
    return matmul(x, dequantize(q, scales, zeros, group_size), bias)


def quantized_matmul_codes(x, codes, zeros, scales, group_size: int, bias=None):
    """Same product from unpacked codes (skips the packing step)."""
    return matmul(x, dequantize(codes, scales, zeros, group_size), bias)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: a bf16 value is the upper half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(v) -> np.ndarray:
    """float64 -> bf16 bit patterns, rounded once to nearest, ties to even (finite values;
    magnitudes past the largest bf16 become infinities).

    bf16 is the upper half of a binary32: 8 exponent bits biased by 127 and 7 stored fraction
    bits. In its normal range (|v| >= 2^-126) it keeps 8 significant bits, so the float64
    significand (53 bits) loses its low 45 bits: they are rounded half to even on the integer
    bit pattern, which carries into the exponent when the significand overflows. Below 2^-126
    the format has fixed spacing: every value is an integer multiple of 2^-133 (exponent -126,
    7 fraction bits), and that integer, rounded half to even, is the bit pattern itself (128
    being the smallest normal, 2^-126).
    """
    d = np.asarray(v, dtype=np.float64)
    u = d.view(np.uint64)
    low = u & np.uint64((1 << 45) - 1)
    q = u >> np.uint64(45)
    half = np.uint64(1 << 44)
    up = (low > half) | ((low == half) & ((q & np.uint64(1)) == np.uint64(1)))
    q = q + up.astype(np.uint64)
    r = (q << np.uint64(45)).view(np.float64)  # exactly representable in bf16 (and binary32)
    normal = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    # Fixed-spacing range: |v| * 2^133 is exact (a power-of-two scaling), np.rint rounds half to even.
    mag = np.abs(d)
    sub = mag < 2.0 ** -126
    units = np.rint(np.where(sub, mag, 0.0) * 2.0 ** 133).astype(np.uint16)  # 0 .. 128
    sign = np.where(np.signbit(d), np.uint16(0x8000), np.uint16(0))
    return np.where(sub, sign | units, normal).astype(np.uint16)


def dequantize_bf16(q: np.ndarray, scales_bf16, zeros_bf16, group_size: int) -> np.ndarray:
    """(K, N) codes -> (K, N) bf16 bit patterns: the exact s * (q - z) rounded once to bf16."""
    return f64_to_bf16(dequantize(q, bf16_to_f64(scales_bf16), bf16_to_f64(zeros_bf16), group_size))


def parity_bound(a: np.ndarray, rel_tol: float = REL_TOL) -> np.ndarray:
    return rel_tol * np.asarray(a, dtype=np.float64) + ABS_TOL


def parity_report(y_dev: np.ndarray, y_ref: np.ndarray, a: np.ndarray, rel_tol: float = REL_TOL) -> dict:
    """Compare a device result (float values, decoded exactly) with the reference.

    ``ok`` holds iff every element is finite and within the bound.
    ``max_ratio`` is the largest |err| / bound; the bound alone is loose, so a
    healthy kernel sits far below 1. ``rel_tol`` is REL_TOL for fp16 data and
    REL_TOL_BF16 for bf16 data.
    """
    yd = np.asarray(y_dev).astype(np.float64)
    err = np.abs(yd - y_ref)
    bound = parity_bound(a, rel_tol)
    finite = np.isfinite(yd)
    ratio = np.where(finite, err / bound, np.inf)
    bad = ~finite | (err > bound)
    return {
        "ok": bool(not bad.any()),
        "violations": int(bad.sum()),
        "nonfinite": int((~finite).sum()),
        "max_ratio": float(ratio.max()) if ratio.size else 0.0,
        "median_ratio": float(np.median(ratio)) if ratio.size else 0.0,
        "max_abs_err": float(err.max()) if err.size else 0.0,
    }


# ---------------------------------------------------------------- strip-major storage order

STRIP_COLS = 16


def to_strips(words: np.ndarray) -> np.ndarray:
    """(rows, N) word plane -> (ceil(N / 16), rows, 16): word (r, n) at [n // 16, r, n % 16], zero padding."""
    rows, N = words.shape
    out = np.zeros(((N + STRIP_COLS - 1) // STRIP_COLS, rows, STRIP_COLS), dtype=words.dtype)
    for n in range(N):
        out[n // STRIP_COLS, :, n % STRIP_COLS] = words[:, n]
    return out


def from_strips(strips: np.ndarray, N: int) -> np.ndarray:
    """Inverse of ``to_strips``: (ceil(N / 16), rows, 16) -> (rows, N)."""
    rows = strips.shape[1]
    out = np.empty((rows, N), dtype=strips.dtype)
    for n in range(N):
        out[:, n] = strips[n // STRIP_COLS, :, n % STRIP_COLS]
    return out
