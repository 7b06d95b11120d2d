"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments before touching the GPU.

No test here launches a kernel: every call below is invalid and must be
refused by host validation (on a machine without a GPU a call that got past
validation would report QMM_ERR_HIP, which these tests treat as a failure).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")


def _lib():
    import weight_only_group_amd as w
    if not os.path.exists(w.LIB_PATH):
        from weight_only_group_amd import build
        build.build()
    return w.library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(
        ["qmm_abi_version", "qmm_status_string", "qmm_last_error", "qmm_pack", "qmm_unpack", "qmm_dequant",
         "qmm_workspace_bytes", "qmm_gemv", "qmm_gemm", "qmm_dequant_bf16", "qmm_gemv_bf16", "qmm_gemm_bf16",
         "qmm_gemv_noalloc",
         "qmm_gemv_plan_info", "qmm_gemm_plan_info", "qmm_strips_bytes", "qmm_to_strips", "qmm_from_strips",
         "qmm_gemv_ex", "qmm_gemm_ex"])


def test_library_exports_every_declared_symbol():
    lib = _lib()
    import weight_only_group_amd as w
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in w.EXPORTS
    # and the shared object's dynamic symbol table has them as plain C names
    raw = ctypes.CDLL(w.LIB_PATH)
    for name in _declared():
        assert getattr(raw, name) is not None


def test_abi_version_and_status_strings():
    lib = _lib()
    assert lib.qmm_abi_version() == 6
    names = [lib.qmm_status_string(i).decode() for i in range(9)]
    assert names == ["QMM_OK", "QMM_ERR_NULL", "QMM_ERR_BITS", "QMM_ERR_SHAPE", "QMM_ERR_GROUP",
                     "QMM_ERR_ALIGN", "QMM_ERR_WORKSPACE", "QMM_ERR_HIP", "QMM_ERR_FLAGS"]
    assert lib.qmm_status_string(99).decode() == "QMM_ERR_UNKNOWN"


def test_workspace_bytes_host_logic():
    lib = _lib()
    # a narrow, deep decode product is split along K and needs partial sums
    n = lib.qmm_workspace_bytes(1, 8192, 64, 4, 128)
    assert n >= 2 * 64 * 4
    assert lib.qmm_workspace_bytes(1, 8192, 64, 4, 128) == n  # deterministic
    assert lib.qmm_workspace_bytes(2, 8192, 64, 4, 128) > n  # grows with M
    # invalid requests need nothing
    for args in ((0, 4096, 4096, 4, 128), (17, 4096, 4096, 4, 128), (1, 4096, 4096, 5, 128),
                 (1, 4000, 4096, 4, 128), (1, 4096, 4100, 4, 128), (1, 4096, 4096, 4, 100)):
        assert lib.qmm_workspace_bytes(*args) == 0, args


# Fake device addresses: aligned and misaligned. They are never dereferenced
# because every call below fails validation first.
A = 0x10000
MIS = 0x10004


def _gemv(lib, suffix="", **kw):
    a = dict(x=A, M=1, K=256, qw=A, qlo=A, z=A, s=A, b=None, N=64, bits=4, gs=128, y=A, ws=A, wsb=1 << 30)
    a.update(kw)
    return getattr(lib, "qmm_gemv" + suffix)(a["x"], a["M"], a["K"], a["qw"], a["qlo"], a["z"], a["s"], a["b"], a["N"], a["bits"],
                        a["gs"], a["y"], a["ws"], a["wsb"], None)


def _gemm(lib, suffix="", **kw):
    a = dict(x=A, M=300, K=256, qw=A, qlo=A, z=A, s=A, b=None, N=64, bits=4, gs=128, y=A)
    a.update(kw)
    return getattr(lib, "qmm_gemm" + suffix)(a["x"], a["M"], a["K"], a["qw"], a["qlo"], a["z"], a["s"], a["b"], a["N"], a["bits"],
                        a["gs"], a["y"], None)


INVALID = [
    ("bits5", dict(bits=5), 2),
    ("bits0", dict(bits=0), 2),
    ("bits6", dict(bits=6), 2),
    ("M0", dict(M=0), 3),
    ("K_not_32", dict(K=48, gs=-1), 3),
    ("N_not_8", dict(N=60), 3),
    ("gs_not_32", dict(gs=48), 4),
    ("gs_not_dividing", dict(K=224, gs=64), 4),
    ("gs_zero", dict(gs=0), 4),
    ("x_null", dict(x=None), 1),
    ("qw_null", dict(qw=None), 1),
    ("lo_null_3bit", dict(bits=3, qlo=None), 1),
    ("scales_null", dict(s=None), 1),
    ("y_null", dict(y=None), 1),
    ("x_misaligned", dict(x=MIS), 5),
    ("zeros_misaligned", dict(z=MIS), 5),
    ("bias_misaligned", dict(b=A + 1), 5),
]
# fp16 and bf16 entry points validate alike.
SUFFIXES = ("", "_bf16")


@pytest.fixture
def host_only():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-validation tests use fake pointers; run them where no GPU is visible")
    return _lib()


@pytest.mark.parametrize("suffix", SUFFIXES)
@pytest.mark.parametrize("name,kw,want", INVALID, ids=[c[0] for c in INVALID])
def test_gemv_rejects_before_launch(host_only, name, kw, want, suffix):
    st = _gemv(host_only, suffix, **kw)
    assert st == want, (name, st, host_only.qmm_last_error())
    assert host_only.qmm_last_error().decode() != ""


@pytest.mark.parametrize("suffix", SUFFIXES)
@pytest.mark.parametrize("name,kw,want", INVALID, ids=[c[0] for c in INVALID])
def test_gemm_rejects_before_launch(host_only, name, kw, want, suffix):
    assert _gemm(host_only, suffix, **kw) == want


def test_gemv_limits(host_only):
    assert _gemv(host_only, M=17) == 3
    # activations too large for the decode kernel's staging: refused (the GEMM takes them)
    assert _gemv(host_only, M=16, K=65536, N=64, gs=-1) == 3
    # arrays of 4 GiB or more are refused by both products
    assert _gemm(host_only, M=1 << 17, K=16384, N=64, gs=-1) == 3
    # a deep, narrow product needs a workspace: too small or missing is refused
    assert host_only.qmm_workspace_bytes(1, 8192, 64, 4, 128) > 16
    assert _gemv(host_only, K=8192, N=64, wsb=16) == 6
    assert _gemv(host_only, K=8192, N=64, ws=None) == 6
    assert _gemv(host_only, K=8192, N=64, ws=MIS) == 5


def test_pack_rejects_before_launch(host_only):
    lib = host_only
    assert lib.qmm_pack(A, 64, 8, 5, A, A, None, None) == 2
    assert lib.qmm_pack(A, 12, 8, 4, A, None, None, None) == 3   # K % 8
    assert lib.qmm_pack(A, 48, 8, 3, A, A, None, None) == 3      # K % 32 for 3-bit
    assert lib.qmm_pack(A, 64, 8, 3, A, None, None, None) == 1   # no 1-bit plane
    assert lib.qmm_pack(None, 64, 8, 4, A, None, None, None) == 1
    assert lib.qmm_pack(A, 0, 8, 4, A, None, None, None) == 3
    assert lib.qmm_unpack(A, None, 64, 8, 3, A, None) == 1
    assert lib.qmm_unpack(A, None, 64, 8, 4, None, None) == 1
    assert lib.qmm_unpack(A, None, 20, 8, 2, A, None) == 3
    assert lib.qmm_pack(A, 48, 8, 1, A, None, None, None) == 3   # K % 32 for 1-bit


@pytest.mark.parametrize("suffix", SUFFIXES)
def test_dequant_rejects_before_launch(host_only, suffix):
    lib = host_only
    dq = getattr(lib, "qmm_dequant" + suffix)
    assert dq(A, A, A, A, 256, 64, 5, 128, A, None) == 2
    assert dq(A, A, A, A, 48, 64, 4, -1, A, None) == 3      # K % 32
    assert dq(A, A, A, A, 256, 64, 4, 48, A, None) == 4     # group size
    assert dq(A, None, A, A, 256, 64, 3, 128, A, None) == 1  # no 1-bit plane
    assert dq(A, A, None, A, 256, 64, 4, 128, A, None) == 1
    assert dq(A, A, A, A, 256, 64, 4, 128, None, None) == 1
    assert dq(A, A, A, A, 256, 64, 4, 128, A + 1, None) == 5  # w not 2-byte aligned
    assert lib.qmm_last_error().decode() != ""


def test_binding_refuses_cpu_tensors():
    import torch
    import weight_only_group_amd as w
    with pytest.raises(ValueError):
        w.qmm_pack(torch.zeros((64, 8), dtype=torch.uint8), 4)
    with pytest.raises((ValueError, TypeError)):
        w.qmm_gemv(torch.zeros((1, 64), dtype=torch.float16), torch.zeros((8, 8), dtype=torch.int32), None,
                   torch.zeros((1, 8), dtype=torch.float16), torch.zeros((1, 8), dtype=torch.float16), 4, -1)
