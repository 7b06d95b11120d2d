"""Host checks of bench.py: its byte counts, the files it hashes for the counter summaries, and its
refusal of more than one GPU (no GPU is used)."""
import os
import subprocess
import sys

import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_workloads():
    # packed words + fp16 scales and zero points + fp16 x + fp16 y
    wl = datagen.WORKLOADS["gemv_m1_k4096_n4096_int4_g128"]
    assert bench.algorithmic_bytes(wl.M, wl.K, wl.N, wl.bits, wl.group_size) == \
        4096 * 4096 // 2 + 2 * 32 * 4096 * 2 + 4096 * 2 + 4096 * 2 == 8929280
    wl = datagen.WORKLOADS["gemv_m1_k2048_n6144_int3_g128"]
    assert bench.algorithmic_bytes(wl.M, wl.K, wl.N, wl.bits, wl.group_size) == \
        2048 * 6144 * 3 // 8 + 2 * 16 * 6144 * 2 + 2048 * 2 + 6144 * 2
    wl = datagen.WORKLOADS["gemm_m2048_k4096_n14336_int8_gchan"]
    assert bench.algorithmic_bytes(wl.M, wl.K, wl.N, wl.bits, wl.group_size) == \
        4096 * 14336 + 2 * 14336 * 2 + 2048 * 4096 * 2 + 2048 * 14336 * 2


def test_kernel_source_files_exist():
    for kind in ("gemv", "gemm"):
        for bits in (1, 2, 3, 4, 8):
            for f in bench.kernel_sources(kind, bits):
                assert os.path.exists(os.path.join(bench.CSRC, f)), f
            assert len(bench.kernel_source_hash(bench.kernel_sources(kind, bits))) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
