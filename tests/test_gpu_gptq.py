"""GPTQModel-format inputs on the GPU against the oracle.

The conversions (packed zero points to (G, N) zero points; 3-bit words of 10
codes to the two 3-bit planes) are integer work and must match the oracle bit
for bit. The product with inputs in that format must meet the element-wise
bound |y - y_ref| <= 2e-3 * sum_k |x_k w_kn| + 1e-3 (9e-3 for bf16 data).
The format is the README's as read in the oracle (value i of a word at bit
offset i * bits, 3-bit words of 10 values with bits 30-31 unused, zero
points packed along N): parity with that reading, unpinned against a layout
the pages print.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def w():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the parity tests")
    import weight_only_group_amd as wm
    wm.library()  # raises if the HIP library is missing
    return wm


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("G,N", [(1, 8), (3, 37), (4, 200), (32, 4104), (64, 11008)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_unpack_qzeros(w, bits, G, N, dtype):
    _say(f"unpack_qzeros bits={bits} G={G} N={N} {dtype}")
    z = datagen.draw_codes(G, N, bits, seed=G * 1000 + N)
    qz = oracle.pack_qzeros(z, bits)
    # every bit of the words is random where the reading leaves it unused (padding, ragged tail)
    used = oracle.pack_qzeros(np.full((G, N), (1 << bits) - 1, dtype=np.uint8), bits).view(np.uint32)
    noise = datagen.draw_codes(G, qz.shape[1] * 4, 8, seed=N).view(np.uint32).reshape(G, qz.shape[1])
    qz_noisy = (qz.view(np.uint32) | (noise & ~used)).view(np.int32)
    got = w.qmm_unpack_qzeros(_t(qz_noisy), bits, N, dtype)
    torch.cuda.synchronize()
    want = oracle.unpack_qzeros(qz, bits, N).astype(np.float32)
    assert got.dtype == dtype and tuple(got.shape) == (G, N)
    assert np.array_equal(got.float().cpu().numpy(), want)


@pytest.mark.parametrize("K,N", [(32, 1), (96, 8), (64, 200), (4096, 136), (2048, 6144)])
def test_repack_3bit10(w, K, N):
    _say(f"repack_3bit10 K={K} N={N}")
    codes = datagen.draw_codes(K, N, 3, seed=K + N)
    w10 = oracle.pack_3bit10(codes)
    qw, qlo = w.qmm_repack_3bit10(_t(w10), K)
    torch.cuda.synchronize()
    hi, lo = oracle.pack_3bit(codes)
    assert np.array_equal(qw.cpu().numpy(), hi)
    assert np.array_equal(qlo.cpu().numpy(), lo)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("M,K,N,gs", [(1, 4096, 512, 128), (5, 2048, 264, -1), (300, 1024, 520, 64)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["fp16", "bf16"])
def test_gptqmodel_product(w, bits, M, K, N, gs, dtype):
    _say(f"gptqmodel_quantized_matmul bits={bits} M={M} K={K} N={N} gs={gs} {dtype}")
    d = datagen.small_case(M, K, N, bits, gs, seed=bits * 7 + M)
    if dtype == torch.bfloat16:
        d = datagen.as_bf16_case(d)
    qweight = oracle.pack_3bit10(d["codes"]) if bits == 3 else oracle.pack_kmajor(d["codes"], bits)
    zeros_f = d["zeros"] if dtype == torch.float16 else oracle.bf16_to_f64(d["zeros"])
    zint = np.asarray(zeros_f, dtype=np.float64)
    assert np.array_equal(zint, np.round(zint))  # integer zero points: the packed format holds nothing else
    qzeros = oracle.pack_qzeros(zint.astype(np.uint8), bits)
    x = _t(d["x"]).view(dtype)
    scales = _t(d["scales"]).view(dtype)
    y = w.gptqmodel_quantized_matmul(x, _t(qweight), _t(qzeros), scales, bits, gs)
    torch.cuda.synchronize()
    s64 = d["scales"] if dtype == torch.float16 else oracle.bf16_to_f64(d["scales"])
    x64 = d["x"] if dtype == torch.float16 else oracle.bf16_to_f64(d["x"])
    y_ref, a = oracle.gptqmodel_quantized_matmul(x64, qweight, qzeros, s64, bits, gs)
    tol = oracle.REL_TOL if dtype == torch.float16 else oracle.REL_TOL_BF16
    rep = oracle.parity_report(y.float().cpu().numpy(), y_ref, a, tol)
    assert rep["ok"], rep
