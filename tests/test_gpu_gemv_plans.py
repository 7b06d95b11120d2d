"""Every compiled variant of the decode product's wave-local kernel against the oracle.

For each variant (code width, columns per lane, waves per block, units per
wave, groups per wave) the smallest shape that the planner sends to it runs
with one activation row and with the most rows the variant takes, in fp16
and in bf16, through qmm_gemv / qmm_gemv_bf16. The zero points rotate over
four kinds: all integers (the one-FMA dequantization is exact), non-integers
everywhere, a column-interleaved mix of small integers, non-integers,
integers above 1024 and non-integers above 1024 (each wave holds all four),
and integers with 1 % of entries made non-integer (waves with and without
the remainder pass in one launch). Some runs add a bias.

The oracle is evaluated on sampled columns: all of the first and the last
strip (the last one ragged) and one column of every strip in between, at a
lane offset that moves from strip to strip, so a strip written to the wrong
place, a wrong lane or a wrong unit, group or row shows. The bound is the
parity bound of the other product tests, with a margin (|err| < 0.35 of it).
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
ZKINDS = ("int", "frac", "mixed", "sparse")


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


def _zeros(kind, G, N, bits, seed):
    rng = np.random.default_rng(seed)
    hi = (1 << bits) - 1
    z = rng.integers(0, hi + 1, size=(G, N)).astype(np.float64)
    if kind == "frac":
        z = rng.uniform(-1.5, hi + 1.5, size=(G, N))
    elif kind == "mixed":
        c = np.arange(N) % 4
        z[:, c == 1] = rng.uniform(-1.5, hi + 1.5, size=(G, int((c == 1).sum())))
        z[:, c == 2] = rng.integers(1025, 1100, size=(G, int((c == 2).sum())))
        z[:, c == 3] = rng.uniform(1024.0, 1030.0, size=(G, int((c == 3).sum())))
    elif kind == "sparse":
        pick = rng.random((G, N)) < 0.01
        z[pick] = rng.uniform(-1.5, hi + 1.5, size=int(pick.sum()))
    return z


def _sample_cols(N, cols):
    strips = (N + cols - 1) // cols
    mid = [s * cols + (s * 5 + 3) % cols for s in range(1, strips - 1)]
    sel = list(range(min(cols, N))) + [c for c in mid if c < N] + list(range((strips - 1) * cols, N))
    return np.unique(np.array(sel, dtype=np.int64))


CASES = cases.wave_cases()
KEYS = list(CASES)


def _id(key):
    return "b{}_v{}_w{}_u{}_g{}".format(*key)


@pytest.mark.parametrize("key", KEYS, ids=[_id(k) for k in KEYS])
def test_wave_variant(gpu, key):
    bits, vec = key[0], key[1]
    K, N, gs, ms = CASES[key]
    idx = KEYS.index(key)
    G = oracle.num_groups(K, gs)
    _say(f"wave variant {_id(key)}: K={K} N={N} gs={gs} M in {ms}")
    codes = datagen.draw_codes(K, N, bits, seed=1000 + idx)
    qw, qlo = gpu.qmm_pack(torch.from_numpy(codes).to(DEV), bits)
    cols = _sample_cols(N, 16 * vec)
    codes_s = codes[:, cols]
    runs = [(M, "fp16", ZKINDS[(idx + i) % 4]) for i, M in enumerate(ms)]
    runs.append((ms[idx % len(ms)], "bf16", ("int", "frac")[idx % 2]))
    for r, (M, dt, zkind) in enumerate(runs):
        p = gpu.gemv_plan_info(M, K, N, bits, gs)
        assert p["kernel"] == 1 and cases.variant(p, bits) == key, (key, M, p)
        seed = 7919 * idx + 31 * r
        x32 = datagen.draw_x_f32(M, K, seed)
        s32 = datagen.draw_scales_f32(G, N, 0.005, 0.05, seed)
        z64 = _zeros(zkind, G, N, bits, seed)
        with_bias = (idx + r) % 3 == 0
        b32 = np.random.default_rng(seed + 1).uniform(-4, 4, size=N).astype(np.float32) if with_bias else None
        _say(f"  M={M} {dt} zeros={zkind} bias={with_bias} seed={seed}")
        if dt == "fp16":
            x, s, z = x32.astype(np.float16), s32.astype(np.float16), z64.astype(np.float16)
            b = None if b32 is None else b32.astype(np.float16)
            t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
            y = gpu.qmm_gemv(t(x), qw, qlo, t(z), t(s), bits, gs, bias=None if b is None else t(b))
            y_ref, a = oracle.quantized_matmul_codes(x, codes_s, z[:, cols], s[:, cols], gs,
                                                     bias=None if b is None else b[cols])
            got = y.cpu().numpy()[:, cols].astype(np.float64)
            rep = oracle.parity_report(got, y_ref, a)
        else:
            xb, sb = datagen.round_to_bf16(x32), datagen.round_to_bf16(s32)
            zb = datagen.round_to_bf16(z64.astype(np.float32))
            bb = None if b32 is None else datagen.round_to_bf16(b32)
            t = lambda u: torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16).to(DEV)
            y = gpu.qmm_gemv(t(xb), qw, qlo, t(zb), t(sb), bits, gs, bias=None if bb is None else t(bb))
            f = oracle.bf16_to_f64
            y_ref, a = oracle.quantized_matmul_codes(f(xb), codes_s, f(zb)[:, cols], f(sb)[:, cols], gs,
                                                     bias=None if bb is None else f(bb)[cols])
            got = f(y.view(torch.int16).cpu().numpy().view(np.uint16)[:, cols])
            rep = oracle.parity_report(got, y_ref, a, rel_tol=oracle.REL_TOL_BF16)
        _say(f"    max|err|/bound={rep['max_ratio']:.4f} median={rep['median_ratio']:.5f} "
             f"violations={rep['violations']} nonfinite={rep['nonfinite']} ({len(cols)} columns)")
        assert rep["ok"], (key, M, dt, zkind, rep)
        assert rep["max_ratio"] < 0.35, (key, M, dt, zkind, rep)
