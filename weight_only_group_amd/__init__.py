"""Python binding of libqmm: the weight-only group-quantized matmul on MI355X.

Argument marshalling only: every step runs in the HIP library (libqmm.so,
built in-tree by ``weight_only_group_amd.build``). PyTorch provides device
memory and the current stream. There is no fallback: if the library is
missing or a tensor is not on a GPU, the call raises.

Functions mirror the C ABI (include/qmm.h):

* ``qmm_pack(codes, bits)`` -> ``(qweight, qweight_lo)``
* ``qmm_unpack(qweight, qweight_lo, K, bits)`` -> codes
* ``qmm_dequant(qweight, qweight_lo, zeros, scales, K, bits, group_size)`` -> (K, N)
* ``qmm_gemv(x, qweight, qweight_lo, zeros, scales, bits, group_size, bias=None)`` (1 <= M <= 16)
* ``qmm_gemv_noalloc(x, qweight, qweight_lo, zeros, scales, bits, group_size, out, bias=None)``:
  the decode product with no workspace (the library's fixed device scratch)
* ``qmm_gemm(x, qweight, qweight_lo, zeros, scales, bits, group_size, bias=None)`` (any M)
* ``quantized_matmul(x, qweight, qzeros, scales, bits, group_size, qweight_lo=None, bias=None)``:
  the functional form, M <= 16 to the GEMV, larger M to the GEMM.

Bit widths 1, 2, 3, 4 and 8. The floating-point data (x, zeros, scales, bias,
the result) are all float16 or all bfloat16; bfloat16 calls the ``_bf16``
entry points of the ABI.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmm.so")

QMM_OK = 0
STATUS_NAMES = {
    0: "QMM_OK", 1: "QMM_ERR_NULL", 2: "QMM_ERR_BITS", 3: "QMM_ERR_SHAPE", 4: "QMM_ERR_GROUP",
    5: "QMM_ERR_ALIGN", 6: "QMM_ERR_WORKSPACE", 7: "QMM_ERR_HIP", 8: "QMM_ERR_FLAGS",
}
# Every symbol the header declares.
EXPORTS = (
    "qmm_abi_version", "qmm_status_string", "qmm_last_error", "qmm_pack", "qmm_unpack", "qmm_dequant",
    "qmm_workspace_bytes", "qmm_gemv", "qmm_gemm", "qmm_dequant_bf16", "qmm_gemv_bf16", "qmm_gemm_bf16",
    "qmm_gemv_noalloc",
    "qmm_gemv_plan_info", "qmm_gemm_plan_info", "qmm_strips_bytes", "qmm_to_strips", "qmm_from_strips",
    "qmm_gemv_ex", "qmm_gemm_ex",
)
ABI_VERSION = 6
QMM_BF16, QMM_STRIPS = 1, 2  # flags of qmm_gemv_ex / qmm_gemm_ex
STRIP_COLS = 16
DTYPES = (torch.float16, torch.bfloat16)
BITS = (1, 2, 3, 4, 8)
GEMV_MAX_M = 16

_lib = None
_lock = threading.Lock()


class QmmError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {detail}")


def _declare(lib):
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.qmm_abi_version.restype = I
    lib.qmm_abi_version.argtypes = []
    lib.qmm_status_string.restype = ctypes.c_char_p
    lib.qmm_status_string.argtypes = [I]
    lib.qmm_last_error.restype = ctypes.c_char_p
    lib.qmm_last_error.argtypes = []
    lib.qmm_pack.restype = I
    lib.qmm_pack.argtypes = [P, I, I, I, P, P, P, P]
    lib.qmm_unpack.restype = I
    lib.qmm_unpack.argtypes = [P, P, I, I, I, P, P]
    lib.qmm_workspace_bytes.restype = SZ
    lib.qmm_workspace_bytes.argtypes = [I, I, I, I, I]
    for suffix in ("", "_bf16"):
        f = getattr(lib, "qmm_dequant" + suffix)
        f.restype, f.argtypes = I, [P, P, P, P, I, I, I, I, P, P]
        f = getattr(lib, "qmm_gemv" + suffix)
        f.restype, f.argtypes = I, [P, I, I, P, P, P, P, P, I, I, I, P, P, SZ, P]
        f = getattr(lib, "qmm_gemm" + suffix)
        f.restype, f.argtypes = I, [P, I, I, P, P, P, P, P, I, I, I, P, P]
    lib.qmm_gemv_noalloc.restype = I
    lib.qmm_gemv_noalloc.argtypes = [P, I, I, P, P, P, P, P, I, I, I, P, P]
    lib.qmm_gemv_plan_info.restype = I
    lib.qmm_gemv_plan_info.argtypes = [I, I, I, I, I, P, I]
    lib.qmm_gemm_plan_info.restype = I
    lib.qmm_gemm_plan_info.argtypes = [I, I, I, I, I, P, I]
    lib.qmm_strips_bytes.restype = SZ
    lib.qmm_strips_bytes.argtypes = [I, I]
    for name in ("qmm_to_strips", "qmm_from_strips"):
        f = getattr(lib, name)
        f.restype, f.argtypes = I, [P, I, I, P, P]
    U = ctypes.c_uint
    lib.qmm_gemv_ex.restype = I
    lib.qmm_gemv_ex.argtypes = [P, I, I, P, P, P, P, P, I, I, I, U, P, P, SZ, P]
    lib.qmm_gemm_ex.restype = I
    lib.qmm_gemm_ex.argtypes = [P, I, I, P, P, P, P, P, I, I, I, U, P, P]
    if lib.qmm_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libqmm ABI version {lib.qmm_abi_version()} does not match the binding's {ABI_VERSION}")
    return lib


def library(path: str | None = None):
    """The loaded libqmm (ctypes.CDLL). Raises if it has not been built."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m weight_only_group_amd.build` "
                    "(there is no fallback implementation)")
            _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(status: int, where: str):
    if status != QMM_OK:
        raise QmmError(status, where, library().qmm_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(t, name, dtype, ndim=2):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def packed_shapes(K: int, N: int, bits: int):
    """Shapes of (qweight, qweight_lo) for K x N codes (qweight_lo None unless bits == 3)."""
    if bits == 3:
        return (K // 16, N), (K // 32, N)
    return (K // (32 // bits), N), None


def qmm_pack(codes: torch.Tensor, bits: int, count_bad: bool = False):
    """(K, N) uint8 codes on the GPU -> (qweight, qweight_lo[, bad_count])."""
    _gpu(codes, "codes", torch.uint8)
    K, N = codes.shape
    shp, shp_lo = packed_shapes(K, N, bits) if bits in BITS else ((1, 1), None)
    dev = codes.device
    qw = torch.empty(shp, dtype=torch.int32, device=dev)
    qlo = torch.empty(shp_lo, dtype=torch.int32, device=dev) if shp_lo else None
    bad = torch.zeros(1, dtype=torch.int32, device=dev) if count_bad else None
    with torch.cuda.device(dev):
        _check(library().qmm_pack(_ptr(codes), K, N, bits, _ptr(qw), _ptr(qlo), _ptr(bad), _stream(dev)), "qmm_pack")
    return (qw, qlo, bad) if count_bad else (qw, qlo)


def qmm_unpack(qweight: torch.Tensor, qweight_lo: torch.Tensor | None, K: int, bits: int) -> torch.Tensor:
    _gpu(qweight, "qweight", torch.int32)
    if qweight_lo is not None:
        _gpu(qweight_lo, "qweight_lo", torch.int32)
    N = qweight.shape[1]
    shp, shp_lo = packed_shapes(K, N, bits) if bits in BITS else (None, None)
    if shp is not None and tuple(qweight.shape) != shp:
        raise ValueError(f"qweight has shape {tuple(qweight.shape)}, expected {shp}")
    if shp_lo is not None and (qweight_lo is None or tuple(qweight_lo.shape) != shp_lo):
        raise ValueError(f"qweight_lo must have shape {shp_lo}")
    dev = qweight.device
    codes = torch.empty((K, N), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        _check(library().qmm_unpack(_ptr(qweight), _ptr(qweight_lo), K, N, bits, _ptr(codes), _stream(dev)),
               "qmm_unpack")
    return codes


def _data_dtype(t, name):
    """The floating-point data type of a call, taken from its first float tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in DTYPES:
        raise TypeError(f"{name} must be float16 or bfloat16 (got {t.dtype})")
    return t.dtype


def _entry(name, dtype):
    return getattr(library(), name + ("_bf16" if dtype == torch.bfloat16 else ""))


def qmm_dequant(qweight, qweight_lo, zeros, scales, K: int, bits: int, group_size: int, out=None):
    """The dequantized weight as (K, N) in the scales' dtype (float16 or
    bfloat16): scale * (q - zero), rounded once."""
    dt = _data_dtype(scales, "scales")
    _gpu(qweight, "qweight", torch.int32)
    if bits == 3:
        if qweight_lo is None:
            raise ValueError("3-bit weights need qweight_lo (the 1-bit plane)")
        _gpu(qweight_lo, "qweight_lo", torch.int32)
    _gpu(zeros, "zeros", dt)
    _gpu(scales, "scales", dt)
    N = qweight.shape[1]
    if bits in BITS:
        shp, shp_lo = packed_shapes(K, N, bits)
        if tuple(qweight.shape) != shp or (shp_lo and tuple(qweight_lo.shape) != shp_lo):
            raise ValueError(f"packed weight shapes {tuple(qweight.shape)} do not match K={K}, N={N}, bits={bits}")
    if zeros.shape != scales.shape or zeros.shape[1] != N:
        raise ValueError("zeros and scales must both be (G, N)")
    dev = qweight.device
    w = torch.empty((K, N), dtype=dt, device=dev) if out is None else _gpu(out, "out", dt)
    if tuple(w.shape) != (K, N):
        raise ValueError(f"out must be ({K}, {N})")
    with torch.cuda.device(dev):
        _check(_entry("qmm_dequant", dt)(_ptr(qweight), _ptr(qweight_lo), _ptr(zeros), _ptr(scales), K, N, bits,
                                         group_size, _ptr(w), _stream(dev)), "qmm_dequant")
    return w


def workspace_bytes(M: int, K: int, N: int, bits: int, group_size: int) -> int:
    return int(library().qmm_workspace_bytes(M, K, N, bits, group_size))


GEMV_PLAN_FIELDS = ("kernel", "vec", "waves", "strips", "ksplit", "units", "groups_per_wave", "xcds", "cus", "one_xcd")


def gemv_plan_info(M: int, K: int, N: int, bits: int, group_size: int) -> dict:
    """The launch plan qmm_gemv takes for this shape on the current device (host only)."""
    info = (ctypes.c_int32 * len(GEMV_PLAN_FIELDS))()
    _check(library().qmm_gemv_plan_info(M, K, N, bits, group_size, ctypes.addressof(info), len(info)),
           "qmm_gemv_plan_info")
    return dict(zip(GEMV_PLAN_FIELDS, list(info)))


GEMM_PLAN_FIELDS = ("bm", "bn", "kgroups", "waves", "blocks", "xcds", "cus")


def gemm_plan_info(M: int, K: int, N: int, bits: int, group_size: int) -> dict:
    """The block tiling qmm_gemm takes for this shape on the current device (host only)."""
    info = (ctypes.c_int32 * len(GEMM_PLAN_FIELDS))()
    _check(library().qmm_gemm_plan_info(M, K, N, bits, group_size, ctypes.addressof(info), len(info)),
           "qmm_gemm_plan_info")
    return dict(zip(GEMM_PLAN_FIELDS, list(info)))


# Zero-filled GEMV workspaces, one per (device, stream); the kernels leave their
# counters at zero, so a workspace is reused call after call on its stream.
_workspaces: dict = {}


def gemv_workspace(device, nbytes: int, stream=None) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    dev = torch.device(device)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    key = (dev.index, s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _check_bias(bias, N, dtype):
    if bias is None:
        return
    _gpu(bias, "bias", dtype, ndim=1)
    if bias.shape[0] != N:
        raise ValueError(f"bias must have N={N} elements")


def strips_shape(rows: int, N: int):
    """Shape of a (rows, N) word plane in the 16-column strip-major layout."""
    return ((N + STRIP_COLS - 1) // STRIP_COLS, rows, STRIP_COLS)


def _check_product_args(x, qweight, qweight_lo, zeros, scales, bits, strips=False):
    dt = _data_dtype(x, "x")
    _gpu(x, "x", dt)
    wdim = 3 if strips else 2
    _gpu(qweight, "qweight", torch.int32, ndim=wdim)
    if bits == 3:
        if qweight_lo is None:
            raise ValueError("3-bit weights need qweight_lo (the 1-bit plane)")
        _gpu(qweight_lo, "qweight_lo", torch.int32, ndim=wdim)
    _gpu(zeros, "zeros", dt)
    _gpu(scales, "scales", dt)
    M, K = x.shape
    N = zeros.shape[1] if strips else qweight.shape[1]
    if bits in BITS:
        shp, shp_lo = packed_shapes(K, N, bits)
        if strips:
            shp, shp_lo = strips_shape(shp[0], N), (strips_shape(shp_lo[0], N) if shp_lo else None)
        if tuple(qweight.shape) != shp or (shp_lo and tuple(qweight_lo.shape) != shp_lo):
            raise ValueError(f"packed weight shapes {tuple(qweight.shape)} do not match K={K}, N={N}, bits={bits}"
                             + (" in 16-column strips" if strips else ""))
    if zeros.shape != scales.shape or zeros.shape[1] != N:
        raise ValueError("zeros and scales must both be (G, N)")
    return M, K, N, dt


def _output(out, M, N, dt, dev):
    if out is None:
        return torch.empty((M, N), dtype=dt, device=dev)
    _gpu(out, "out", dt)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be ({M}, {N})")
    return out


def _flags(dt, strips):
    return (QMM_BF16 if dt == torch.bfloat16 else 0) | (QMM_STRIPS if strips else 0)


def qmm_gemv(x, qweight, qweight_lo, zeros, scales, bits: int, group_size: int, out=None, workspace=None,
             bias=None, strips: bool = False):
    """y = x @ dequantize(W) (+ bias) for 1 <= M <= 16; returns (M, N) in x's dtype. With
    ``strips=True`` the packed planes are in the 16-column strip-major layout of qmm_to_strips."""
    M, K, N, dt = _check_product_args(x, qweight, qweight_lo, zeros, scales, bits, strips)
    _check_bias(bias, N, dt)
    dev = x.device
    y = _output(out, M, N, dt, dev)
    nbytes = workspace_bytes(M, K, N, bits, group_size) if M <= GEMV_MAX_M else 0
    ws = workspace if workspace is not None else gemv_workspace(dev, nbytes)
    with torch.cuda.device(dev):
        args = (_ptr(x), M, K, _ptr(qweight), _ptr(qweight_lo), _ptr(zeros), _ptr(scales), _ptr(bias), N, bits,
                group_size)
        tail = (_ptr(y), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
        if strips:
            _check(library().qmm_gemv_ex(*args, _flags(dt, True), *tail), "qmm_gemv_ex")
        else:
            _check(_entry("qmm_gemv", dt)(*args, *tail), "qmm_gemv")
    return y


def qmm_gemv_noalloc(x, qweight, qweight_lo, zeros, scales, bits: int, group_size: int, out, bias=None):
    """qmm_gemv into a caller-given ``out`` (M, N) without any workspace: the library's own fixed
    device scratch serves the split-K plans (float16 data; shapes needing more than its 4 MiB are
    refused). Calls that overlap in time on one GPU must not use it concurrently."""
    M, K, N, dt = _check_product_args(x, qweight, qweight_lo, zeros, scales, bits)
    if dt != torch.float16:
        raise TypeError("qmm_gemv_noalloc takes float16 data")
    _check_bias(bias, N, dt)
    dev = x.device
    y = _output(out, M, N, dt, dev)
    with torch.cuda.device(dev):
        _check(library().qmm_gemv_noalloc(_ptr(x), M, K, _ptr(qweight), _ptr(qweight_lo), _ptr(zeros), _ptr(scales),
                                          _ptr(bias), N, bits, group_size, _ptr(y), _stream(dev)),
               "qmm_gemv_noalloc")
    return y


def qmm_gemm(x, qweight, qweight_lo, zeros, scales, bits: int, group_size: int, out=None, bias=None,
             strips: bool = False):
    """y = x @ dequantize(W) (+ bias) for any M on the matrix cores; returns (M, N) in x's dtype.
    ``strips=True``: the packed planes are in the strip-major layout of qmm_to_strips."""
    M, K, N, dt = _check_product_args(x, qweight, qweight_lo, zeros, scales, bits, strips)
    _check_bias(bias, N, dt)
    dev = x.device
    y = _output(out, M, N, dt, dev)
    with torch.cuda.device(dev):
        args = (_ptr(x), M, K, _ptr(qweight), _ptr(qweight_lo), _ptr(zeros), _ptr(scales), _ptr(bias), N, bits,
                group_size)
        if strips:
            _check(library().qmm_gemm_ex(*args, _flags(dt, True), _ptr(y), _stream(dev)), "qmm_gemm_ex")
        else:
            _check(_entry("qmm_gemm", dt)(*args, _ptr(y), _stream(dev)), "qmm_gemm")
    return y


def qmm_to_strips(words: torch.Tensor, out=None) -> torch.Tensor:
    """A (rows, N) int32 word plane -> its 16-column strip-major form (ceil(N / 16), rows, 16):
    word (r, n) at [n // 16, r, n % 16], the last strip's columns past N zero. Load-time work."""
    _gpu(words, "words", torch.int32)
    rows, N = words.shape
    shape = strips_shape(rows, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=words.device)
    else:
        _gpu(out, "out", torch.int32, ndim=3)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {shape}")
    with torch.cuda.device(words.device):
        _check(library().qmm_to_strips(_ptr(words), rows, N, _ptr(out), _stream(words.device)), "qmm_to_strips")
    return out


def qmm_from_strips(strips: torch.Tensor, N: int) -> torch.Tensor:
    """Inverse of qmm_to_strips: (ceil(N / 16), rows, 16) -> (rows, N)."""
    _gpu(strips, "strips", torch.int32, ndim=3)
    S, rows, c = strips.shape
    if (S, c) != strips_shape(rows, N)[::2]:
        raise ValueError(f"strips {tuple(strips.shape)} do not hold a plane of N={N} columns")
    out = torch.empty((rows, N), dtype=torch.int32, device=strips.device)
    with torch.cuda.device(strips.device):
        _check(library().qmm_from_strips(_ptr(strips), rows, N, _ptr(out), _stream(strips.device)), "qmm_from_strips")
    return out


def quantized_matmul(x, qweight, qzeros, scales, bits: int, group_size: int, qweight_lo=None, bias=None):
    """output = x @ dequantize(qweight) (+ bias), in the argument order of the functional API.

    ``qzeros`` are the (G, N) zero points, in x's dtype (float16 or bfloat16); M <= 16 runs the decode GEMV
    (the GEMM when the GEMV's staging limits reject the shape), larger M the
    prefill GEMM.
    """
    if x.dim() != 2:
        raise ValueError("x must be (M, K)")
    if x.shape[0] <= GEMV_MAX_M:
        try:
            return qmm_gemv(x, qweight, qweight_lo, qzeros, scales, bits, group_size, bias=bias)
        except QmmError as e:
            if e.status != 3:  # QMM_ERR_SHAPE: shape beyond the decode kernel's staging limits
                raise
    return qmm_gemm(x, qweight, qweight_lo, qzeros, scales, bits, group_size, bias=bias)
