"""The seeded input generator: reproducible, with the stated shapes and distributions."""
import hashlib

import numpy as np

import datagen


def _digest(d):
    h = hashlib.sha256()
    for k in sorted(d):
        h.update(k.encode())
        h.update(np.ascontiguousarray(d[k]).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    w = datagen.WORKLOADS["gemv_m1_k512_n256_int4_g128"]
    assert _digest(datagen.generate(w)) == _digest(datagen.generate(w))
    assert _digest(datagen.generate(w, seed=1)) != _digest(datagen.generate(w))


def test_arrays_independent_of_row_count():
    w = datagen.WORKLOADS["gemm_m8_k4096_n11008_int2_g64"]
    a = datagen.generate(w, M=2)
    b = datagen.generate(w)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    assert np.array_equal(a["x"], datagen.draw_x(2, w.K, w.seed))


def test_workload_shapes_and_ranges():
    for name, w in datagen.WORKLOADS.items():
        if w.M * w.K * w.N > 1e9:
            d = datagen.generate(w, M=4)  # rows sampled for the prefill-sized product
        else:
            d = datagen.generate(w)
        G = w.groups
        assert d["codes"].shape == (w.K, w.N) and d["codes"].dtype == np.uint8
        assert d["codes"].max() <= (1 << w.bits) - 1
        assert d["zeros"].shape == (G, w.N) and d["zeros"].dtype == np.float16
        z = d["zeros"].astype(np.float64)
        assert np.all(z == np.round(z)) and z.min() >= w.zero_range[0] and z.max() <= w.zero_range[1]
        s = d["scales"].astype(np.float64)
        assert d["scales"].dtype == np.float16 and s.min() >= w.scale_range[0] * 0.999 and s.max() <= w.scale_range[1] * 1.001
        assert d["x"].dtype == np.float16 and d["x"].shape[1] == w.K
        xs = d["x"].astype(np.float64)
        assert abs(xs.mean()) < 0.1 and 0.9 < xs.std() < 1.1, name
        # every code value occurs
        assert len(np.unique(d["codes"][:64])) == 1 << w.bits, name


def test_bf16_inputs_are_nearest_even_roundings():
    """bf16 inputs are the draws rounded once to bf16 (compared with the oracle's own rounding)."""
    import oracle
    d = datagen.small_case(2, 64, 16, 4, 32, seed=3)
    b = datagen.as_bf16_case(d)
    assert np.array_equal(b["x"], oracle.f64_to_bf16(d["x_f32"].astype(np.float64)))
    assert np.array_equal(b["scales"], oracle.f64_to_bf16(d["scales_f32"].astype(np.float64)))
    assert np.array_equal(oracle.bf16_to_f64(b["zeros"]), d["zeros"].astype(np.float64))  # small integers: exact
