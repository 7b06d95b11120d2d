"""qmm_gemv_noalloc (the decode product without a workspace, for callers that
cannot allocate) against qmm_gemv with a workspace, through the C ABI.

Both entry points run the same kernels in the same order, so their outputs
must agree bit for bit; each is also within the parity rule of the CPU
oracle. Two calls in a row on the library's shared scratch, the second on a
smaller input, check that nothing from the first call leaks into the second
(the arrival counters are left at zero, the partial sums are overwritten).
The shapes are split along K, so the scratch is really used.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
QMM_ERR_WORKSPACE = 6


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required")
    import weight_only_group_amd as mod
    mod.library()
    return mod


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(w, M, K, N, bits, gs, seed):
    d = datagen.small_case(M, K, N, bits, gs, seed=seed)
    qw, qlo = w.qmm_pack(torch.from_numpy(d["codes"]).to(DEV), bits)
    x, z, s = (torch.from_numpy(d[k]).to(DEV) for k in ("x", "zeros", "scales"))
    return d, x, qw, qlo, z, s


def _call_noalloc(w, x, qw, qlo, z, s, bits, gs, y, bias=None):
    """The raw C entry point (ctypes), on the current stream."""
    M, K = x.shape
    N = qw.shape[1]
    lib = w.library()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    return lib.qmm_gemv_noalloc(p(x), M, K, p(qw), p(qlo), p(z), p(s), p(bias), N, bits, gs, p(y),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("first,second", [
    ((4, 8192, 512, 4, 128), (1, 4096, 256, 4, 128)),
    ((16, 8192, 1024, 4, 128), (2, 4096, 256, 3, 128)),
    ((16, 32768, 2048, 4, -1), (8, 2048, 512, 2, 64)),
])
def test_noalloc_matches_workspace_entry(w, first, second):
    outs = []
    for i, (M, K, N, bits, gs) in enumerate((first, second)):
        need = w.workspace_bytes(M, K, N, bits, gs)
        assert 0 < need <= 4 << 20, (M, K, N, need)  # split along K, within the scratch
        _say(f"noalloc call {i}: M={M} K={K} N={N} bits={bits} gs={gs} (plan scratch {need} B)")
        d, x, qw, qlo, z, s = _case(w, M, K, N, bits, gs, seed=31 + i + M + N)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=DEV)
        st = _call_noalloc(w, x, qw, qlo, z, s, bits, gs, y)
        assert st == 0, w.library().qmm_last_error().decode()
        torch.cuda.synchronize()
        y_ws = w.qmm_gemv(x, qw, qlo, z, s, bits, gs)
        torch.cuda.synchronize()
        got, want = y.cpu().numpy(), y_ws.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), \
            f"call {i}: {np.count_nonzero(got.view(np.uint16) != want.view(np.uint16))} elements differ"
        y_ref, a = oracle.quantized_matmul_codes(d["x"], d["codes"], d["zeros"], d["scales"], gs)
        rep = oracle.parity_report(got, y_ref, a)
        assert rep["ok"] and rep["max_ratio"] < 0.35, rep
        outs.append(got)


def test_noalloc_repeat_is_bitwise_stable(w):
    """The same call twice on the shared scratch gives the same bits (counters back at zero)."""
    M, K, N, bits, gs = 4, 8192, 512, 4, 128
    _say(f"noalloc repeat M={M} K={K} N={N}")
    d, x, qw, qlo, z, s = _case(w, M, K, N, bits, gs, seed=77)
    ys = []
    for _ in range(3):
        y = torch.empty((M, N), dtype=torch.float16, device=DEV)
        assert _call_noalloc(w, x, qw, qlo, z, s, bits, gs, y) == 0
        torch.cuda.synchronize()
        ys.append(y.cpu().numpy().view(np.uint16))
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[1], ys[2])


def test_noalloc_refuses_shapes_beyond_its_scratch(w):
    """A plan needing more than the 4 MiB scratch is refused on the host; nothing is launched."""
    M, K, N, bits, gs = 16, 16384, 8192, 4, -1
    assert w.workspace_bytes(M, K, N, bits, gs) > 4 << 20
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    qw = torch.zeros((K // 8, N), dtype=torch.int32, device=DEV)
    z = torch.zeros((1, N), dtype=torch.float16, device=DEV)
    s = torch.zeros((1, N), dtype=torch.float16, device=DEV)
    y = torch.full((M, N), 7.0, dtype=torch.float16, device=DEV)
    st = _call_noalloc(w, x, qw, None, z, s, bits, gs, y)
    assert st == QMM_ERR_WORKSPACE, st
    assert "scratch" in w.library().qmm_last_error().decode()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())  # output untouched
