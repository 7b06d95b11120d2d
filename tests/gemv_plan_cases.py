"""Shapes that reach each variant of the decode product's wave-local kernel.

A variant is the tuple (bits, columns per lane, waves per block, 32-row units
per wave, groups per wave) that qmm_gemv_plan_info reports for a shape sent to
that kernel; each is a separate compiled instance (for one activation row and
for several, fp16 and bf16). ``wave_cases()`` finds, on a small grid of
candidate shapes, the smallest (K * N) one per variant; ``full_sweep()``
walks a much wider grid, so a test can show that the small grid misses no
variant the planner can reach. Host only: nothing is launched.
"""
import functools

import weight_only_group_amd as w

BITS = (1, 2, 3, 4, 8)
CAND_K = (512, 1024, 2048, 4096, 8192)
CAND_GS = (-1, 32, 64, 128, 256)
# Up to one strip of 16 columns per CU (1024: few enough strips that short K
# is split; 2056: enough that it is not), up to 2 and up to 4 times that,
# each but the first with a ragged last strip; and wide enough for 3- and
# 8-bit codes at 4 columns per lane to need no split along K.
CAND_N = (1024, 2056, 4104, 8200, 16392)
CAND_M = (1, 8, 16)


def variant(plan: dict, bits: int):
    return (bits, plan["vec"], plan["waves"], plan["units"], plan["groups_per_wave"])


def plan(M, K, N, bits, gs):
    try:
        return w.gemv_plan_info(M, K, N, bits, gs)
    except w.QmmError:
        return None


@functools.lru_cache(maxsize=None)
def wave_cases():
    """{variant: (K, N, gs, Ms)}: the smallest candidate shape per variant, with the
    activation row counts to run it at (1 if the variant takes one row, and the
    largest M <= 16 that keeps the shape on the same variant)."""
    best = {}
    for bits in BITS:
        for K in CAND_K:
            for gs in CAND_GS:
                if gs != -1 and K % gs:
                    continue
                for N in CAND_N:
                    for M0 in CAND_M:
                        p = plan(M0, K, N, bits, gs)
                        if p is None or p["kernel"] != 1:
                            continue
                        key = variant(p, bits)
                        if key not in best or K * N < best[key][0] * best[key][1]:
                            best[key] = (K, N, gs)
    out = {}
    for key, (K, N, gs) in sorted(best.items()):
        bits = key[0]
        ms = []
        p1 = plan(1, K, N, bits, gs)
        if p1 is not None and p1["kernel"] == 1 and variant(p1, bits) == key:
            ms.append(1)
        for M in range(16, 1, -1):
            p = plan(M, K, N, bits, gs)
            if p is not None and p["kernel"] == 1 and variant(p, bits) == key:
                ms.append(M)
                break
        out[key] = (K, N, gs, tuple(ms))
    return out


def full_sweep():
    """Variants reached over K = 256 .. 16384 (step 256), eight group sizes, eleven
    column counts and four row counts."""
    seen = set()
    for bits in BITS:
        for K in range(256, 16385, 256):
            for gs in (-1, 32, 64, 128, 256, 512, 1024, 2048):
                if gs != -1 and K % gs:
                    continue
                for N in (8, 1024, 4096, 4104, 6144, 8192, 8200, 11008, 14336, 28672, 65536):
                    for M in (1, 2, 8, 16):
                        p = plan(M, K, N, bits, gs)
                        if p is not None and p["kernel"] == 1:
                            seen.add(variant(p, bits))
    return seen
