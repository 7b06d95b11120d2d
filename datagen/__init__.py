"""Seeded synthetic inputs for the weight-only group-quantized matmul.

Shared by the oracle side and the device side, and nothing else: this module
draws integer codes, zero points, scales and activations with the
distributions of the named workloads. It holds none of the method's
arithmetic (no packing, no dequantization, no product).

Every array has its own PCG64 stream keyed by (seed, array tag), so the
values of one array never depend on the size of another or on draw order.
Floating-point draws are rounded to IEEE binary16 (round to nearest even) by
numpy; every consumer uses the stored fp16 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Tags keep the four streams of one workload independent of each other.
_TAG_CODES, _TAG_ZEROS, _TAG_SCALES, _TAG_X = 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """Shape and value distributions of one synthetic problem.

    ``group_size == -1`` means one group spanning all of K (per output column).
    Codes are uniform integers in [0, 2**bits - 1]; zero points are uniform
    integers in ``zero_range`` stored as fp16; scales are fp16 draws of a
    uniform real in ``scale_range``; activations are fp16 draws of N(0, 1).
    """

    name: str
    M: int
    K: int
    N: int
    bits: int
    group_size: int
    zero_range: tuple = (0, 15)
    scale_range: tuple = (0.005, 0.02)
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def groups(self) -> int:
        return 1 if self.group_size == -1 else self.K // self.group_size


# The five named workloads. The first is the small case every check can afford
# in full; the second is the decode projection the throughput figure is quoted
# on; the last is the prefill-sized product.
WORKLOADS = {
    w.name: w
    for w in (
        Workload("gemv_m1_k512_n256_int4_g128", 1, 512, 256, 4, 128, (0, 15), (0.005, 0.02),
                 note="small decode product"),
        Workload("gemv_m1_k4096_n4096_int4_g128", 1, 4096, 4096, 4, 128, (0, 15), (0.005, 0.02),
                 note="one transformer projection, decode"),
        Workload("gemv_m1_k2048_n6144_int3_g128", 1, 2048, 6144, 3, 128, (0, 7), (0.01, 0.04),
                 note="3-bit as a 2-bit plane plus a 1-bit plane"),
        Workload("gemm_m8_k4096_n11008_int2_g64", 8, 4096, 11008, 2, 64, (0, 3), (0.02, 0.08),
                 note="small batch, 2-bit"),
        Workload("gemm_m2048_k4096_n14336_int8_gchan", 2048, 4096, 14336, 8, -1, (96, 160), (0.001, 0.004),
                 note="prefill, 8-bit, one scale and zero per column"),
    )
}

# The decode workload the throughput figure is quoted on, and the prefill one.
HEADLINE_GEMV = "gemv_m1_k4096_n4096_int4_g128"
HEADLINE_GEMM = "gemm_m2048_k4096_n14336_int8_gchan"


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tag)])))


def draw_codes(K: int, N: int, bits: int, seed: int = 0, high: int | None = None) -> np.ndarray:
    """(K, N) uint8 codes, uniform on [0, high] (default 2**bits - 1)."""
    hi = (1 << bits) - 1 if high is None else high
    return _rng(seed, _TAG_CODES).integers(0, hi + 1, size=(K, N), dtype=np.uint8)


def draw_zeros(G: int, N: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """(G, N) fp16 zero points, uniform integers on [lo, hi]."""
    z = _rng(seed, _TAG_ZEROS).integers(lo, hi + 1, size=(G, N), dtype=np.int64)
    return z.astype(np.float16)


def draw_scales_f32(G: int, N: int, lo: float, hi: float, seed: int = 0) -> np.ndarray:
    """(G, N) float32 draws of a uniform real on [lo, hi)."""
    return _rng(seed, _TAG_SCALES).uniform(lo, hi, size=(G, N)).astype(np.float32)


def draw_scales(G: int, N: int, lo: float, hi: float, seed: int = 0) -> np.ndarray:
    """(G, N) fp16 scales, a uniform real on [lo, hi) rounded to fp16."""
    return _rng(seed, _TAG_SCALES).uniform(lo, hi, size=(G, N)).astype(np.float16)


def draw_x_f32(M: int, K: int, seed: int = 0) -> np.ndarray:
    """(M, K) float32 draws of N(0, 1)."""
    return _rng(seed, _TAG_X).standard_normal(size=(M, K), dtype=np.float32)


def draw_x(M: int, K: int, seed: int = 0) -> np.ndarray:
    """(M, K) fp16 activations, N(0, 1) rounded to fp16."""
    return draw_x_f32(M, K, seed).astype(np.float16)


def generate(w: Workload | str, seed: int | None = None, M: int | None = None) -> dict:
    """All inputs of one workload as numpy arrays.

    Returns ``codes`` (K, N) uint8, ``zeros`` and ``scales`` (G, N) float16 and
    ``x`` (M, K) float16, plus ``scales_f32`` and ``x_f32``, the same draws
    before their rounding to fp16. ``M`` overrides the workload's row count (used for
    row-sampled checks of large products).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    s = w.seed if seed is None else seed
    m = w.M if M is None else M
    G = w.groups
    x32 = draw_x_f32(m, w.K, s)
    s32 = draw_scales_f32(G, w.N, w.scale_range[0], w.scale_range[1], s)
    return {
        "codes": draw_codes(w.K, w.N, w.bits, s),
        "zeros": draw_zeros(G, w.N, w.zero_range[0], w.zero_range[1], s),
        "scales": draw_scales(G, w.N, w.scale_range[0], w.scale_range[1], s),
        "x": x32.astype(np.float16),
        # the same draws before their rounding to fp16 (for bf16 cases)
        "scales_f32": s32,
        "x_f32": x32,
    }


def round_to_bf16(values) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), nearest even (the inputs' storage format)."""
    u = np.asarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def as_bf16_case(d: dict) -> dict:
    """The same draws stored as bf16: x, scales and zero points re-rounded from the draws'
    float32 values (integer zero points stay exact up to 256)."""
    return {
        "codes": d["codes"],
        "zeros": round_to_bf16(d["zeros"].astype(np.float32)),
        "scales": round_to_bf16(d["scales_f32"]),
        "x": round_to_bf16(d["x_f32"]),
    }


def small_case(M: int, K: int, N: int, bits: int, group_size: int, seed: int = 0,
               zero_range: tuple | None = None, scale_range: tuple = (0.005, 0.05)) -> dict:
    """Inputs of an arbitrary small shape with the workloads' distributions."""
    hi = (1 << bits) - 1
    zr = (0, hi) if zero_range is None else zero_range
    w = Workload(f"case_m{M}_k{K}_n{N}_b{bits}_g{group_size}", M, K, N, bits, group_size, zr, scale_range, seed)
    return generate(w)
