"""Host checks of the decode product's launch plans (qmm_gemv_plan_info).

Each plan must tile the problem exactly: the wave-local kernel gives every
wave the same number of 32-row units and covers all of K in one block per
column strip; the split kernel's blocks along K cover K with no block empty.
The small grid of shapes the GPU tests run must reach every variant of the
wave-local kernel that a much wider sweep reaches. No kernel is launched.
"""
import os

import pytest

import gemv_plan_cases as cases


def _lib():
    import weight_only_group_amd as w
    if not os.path.exists(w.LIB_PATH):
        from weight_only_group_amd import build
        build.build()
    return w


def _words_per_unit(bits):
    return 2 if bits in (3, 8) else 1


@pytest.mark.parametrize("bits", cases.BITS)
def test_plans_tile_the_problem(bits):
    w = _lib()
    for K in (32, 96, 256, 512, 1024, 2080, 4096, 8192, 14336, 16384):
        for gs in (-1, 32, 64, 128, 1024):
            if gs != -1 and K % gs:
                continue
            for N in (8, 136, 1024, 4096, 4104, 8200, 14336, 65536):
                for M in (1, 3, 16):
                    p = cases.plan(M, K, N, bits, gs)
                    if p is None:  # beyond the staging limits: qmm_gemv refuses it too
                        continue
                    U = K // 32
                    cols = 16 * p["vec"]
                    assert p["vec"] in (1, 2, 4)
                    assert p["strips"] == (N + cols - 1) // cols
                    assert p["xcds"] >= 1 and p["cus"] >= 1
                    # all strips on XCD 0: the wave kernel, at most one strip per CU of an XCD,
                    # at most 1 MiB of weight words
                    small = p["strips"] <= p["cus"] // p["xcds"] and K * N * bits // 8 <= 1 << 20
                    assert p["one_xcd"] == int(p["kernel"] == 1 and p["xcds"] > 1 and small)
                    if p["kernel"] == 1:
                        assert p["ksplit"] == 1
                        assert p["waves"] * p["units"] == U
                        assert p["groups_per_wave"] in (1, 2, 4)
                        assert p["units"] * _words_per_unit(bits) * p["vec"] <= 32  # weight words per lane
                        assert M * U * 4 <= 4 * 64 * p["waves"]  # activation slots within the staging area
                        upg = U if gs == -1 else gs // 32
                        if p["groups_per_wave"] > 1:
                            assert p["units"] == p["groups_per_wave"] * upg
                        else:
                            assert gs == -1 or upg % p["units"] == 0
                    else:
                        assert p["kernel"] == 0 and p["groups_per_wave"] == 0
                        ks, upb = p["ksplit"], p["units"]
                        assert 1 <= ks <= 16
                        assert ks * upb >= U > (ks - 1) * upb  # K covered, no block empty
                        assert (w.workspace_bytes(M, K, N, bits, gs) > 0) == (ks > 1)


def test_candidate_grid_reaches_every_wave_variant():
    _lib()
    found = set(cases.wave_cases())
    swept = cases.full_sweep()
    assert swept <= found, sorted(swept - found)
    # every code width appears at every column width
    for bits in cases.BITS:
        assert {v[1] for v in found if v[0] == bits} == {1, 2, 4}, bits


def test_wave_cases_run_on_the_variant_they_name():
    _lib()
    for key, (K, N, gs, ms) in cases.wave_cases().items():
        assert ms, key
        for M in ms:
            p = cases.plan(M, K, N, key[0], gs)
            assert p["kernel"] == 1 and cases.variant(p, key[0]) == key, (key, M)


def test_headline_decode_shapes_take_the_wave_kernel():
    import datagen
    w = _lib()
    for name, wl in datagen.WORKLOADS.items():
        if wl.M > 16:
            continue
        p = w.gemv_plan_info(wl.M, wl.K, wl.N, wl.bits, wl.group_size)
        assert p["kernel"] == 1, (name, p)


def test_plan_info_rejects_what_qmm_gemv_rejects():
    w = _lib()
    for args in ((0, 4096, 4096, 4, 128), (17, 4096, 4096, 4, 128), (1, 4096, 4096, 5, 128),
                 (1, 4000, 4096, 4, 128), (1, 4096, 4100, 4, 128), (1, 4096, 4096, 4, 100),
                 (1, 4096, (1 << 20) + 8, 4, 128)):
        with pytest.raises(w.QmmError):
            w.gemv_plan_info(*args)
    lib = w.library()
    assert lib.qmm_gemv_plan_info(1, 4096, 4096, 4, 128, None, 4) == 1  # QMM_ERR_NULL
    assert lib.qmm_gemv_plan_info(1, 4096, 4096, 4, 128, None, 0) == 0  # nothing to write


def test_gemm_block_tiles():
    w = _lib()
    import datagen
    wl = datagen.WORKLOADS[datagen.HEADLINE_GEMM]
    p = w.gemm_plan_info(wl.M, wl.K, wl.N, wl.bits, wl.group_size)
    assert (p["bm"], p["bn"], p["kgroups"], p["waves"], p["blocks"]) == (256, 256, 1, 8, 8 * 56)
    for M, K, N in ((1, 32, 8), (300, 512, 264), (4100, 544, 4104), (65536, 64, 8), (16, 32, 65536)):
        p = w.gemm_plan_info(M, K, N, 4, -1)
        assert p["blocks"] == ((M + p["bm"] - 1) // p["bm"]) * ((N + p["bn"] - 1) // p["bn"])
        # the largest tile whose grid still covers the CUs
        if p["bm"] < 256:
            assert ((M + 255) // 256) * ((N + 255) // 256) < p["cus"]
        assert p["waves"] in (8, 12, 16) and p["kgroups"] in (1, 2, 4, 6)
    for args in ((0, 64, 64, 4, -1), (1, 40, 64, 4, -1), (1, 64, 60, 4, -1), (1, 64, 64, 6, -1), (1, 64, 64, 4, 48)):
        with pytest.raises(w.QmmError):
            w.gemm_plan_info(*args)


def test_one_xcd_boundary():
    """32 strips of a short-K product run on XCD 0 alone, 33 take every XCD; the rule needs the
    wave kernel and at most 1 MiB of weight words (8 XCDs of 32 CUs: the default topology
    without a device, and MI355X's)."""
    w = _lib()
    on = w.gemv_plan_info(1, 512, 512, 4, 128)
    if on["xcds"] != 8 or on["cus"] != 256:
        pytest.skip("the boundary below assumes 8 XCDs of 32 CUs")
    assert on["kernel"] == 1 and on["strips"] == 32 and on["one_xcd"] == 1
    off = w.gemv_plan_info(1, 512, 520, 4, 128)
    assert off["kernel"] == 1 and off["strips"] == 33 and off["one_xcd"] == 0
    split = w.gemv_plan_info(1, 4096, 512, 4, 128)  # few strips, long K: blocks split along K
    assert split["kernel"] == 0 and split["one_xcd"] == 0

