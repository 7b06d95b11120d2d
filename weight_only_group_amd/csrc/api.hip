// C ABI: argument validation, error reporting and dispatch to the kernels.
// Every check runs on the host before anything is enqueued; no HIP call is
// made for an invalid request.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/qmm.h"
#include "common.h"

namespace qmm {

// Read once per device: the plans size their grids by the CU count and lay
// out strips by the XCD count. Without a device (host-only use of
// qmm_workspace_bytes) the MI355X values are taken.
DeviceTopo device_topology() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static DeviceTopo cache[kMaxDev] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return DeviceTopo{256, 8};
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev].cus == 0) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds <= 0) xcds = 8;
    (void)hipGetLastError();
    cache[dev] = DeviceTopo{cus, xcds};
  }
  return cache[dev];
}

}  // namespace qmm

namespace {

thread_local char g_last_error[512] = "";

qmm_status fail(qmm_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

qmm_status ok() {
  g_last_error[0] = '\0';
  return QMM_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

bool bits_ok(int bits) { return bits == 1 || bits == 2 || bits == 3 || bits == 4 || bits == 8; }

// Codes per word of the plane that sets the K granularity.
int k_multiple(int bits) { return bits == 3 ? 32 : 32 / bits; }

qmm_status check_packing(int K, int N, int bits, const void* qweight, const void* qweight_lo) {
  if (!bits_ok(bits)) return fail(QMM_ERR_BITS, "bits=%d is not one of 1, 2, 3, 4, 8", bits);
  if (K < 1 || N < 1) return fail(QMM_ERR_SHAPE, "K=%d and N=%d must be >= 1", K, N);
  if (K % k_multiple(bits)) return fail(QMM_ERR_SHAPE, "K=%d must be a multiple of %d for %d-bit codes", K, k_multiple(bits), bits);
  if (qweight == nullptr) return fail(QMM_ERR_NULL, "qweight is NULL");
  if (bits == 3 && qweight_lo == nullptr) return fail(QMM_ERR_NULL, "qweight_lo (1-bit plane) is NULL for 3-bit codes");
  return QMM_OK;
}

qmm_status check_group(int K, int group_size) {
  if (group_size != -1 && (group_size <= 0 || group_size % 32 || K % group_size))
    return fail(QMM_ERR_GROUP, "group_size=%d must be -1 or a positive multiple of 32 dividing K=%d", group_size, K);
  return QMM_OK;
}

// The shape rules every product applies (and the plan queries with them).
qmm_status check_product_shape(int M, int K, int N, int bits, int group_size, int max_m) {
  if (!bits_ok(bits)) return fail(QMM_ERR_BITS, "bits=%d is not one of 1, 2, 3, 4, 8", bits);
  if (M < 1 || M > max_m) return fail(QMM_ERR_SHAPE, "M=%d must be in [1, %d]", M, max_m);
  if (K < 32 || K % 32) return fail(QMM_ERR_SHAPE, "K=%d must be a positive multiple of 32", K);
  if (N < 8 || N % 8) return fail(QMM_ERR_SHAPE, "N=%d must be a positive multiple of 8", N);
  {
    const qmm_status gs = check_group(K, group_size);
    if (gs != QMM_OK) return gs;
  }
  // Kernels address x, the packed planes, scales and zero points with 32-bit
  // byte offsets.
  const unsigned long long lim = 1ull << 32;
  const unsigned long long groups = group_size == -1 ? 1ull : (unsigned long long)(K / group_size);
  if ((unsigned long long)M * K * 2 >= lim || (unsigned long long)K * N * (bits == 3 ? 2 : bits) / 8 >= lim ||
      groups * N * 2 >= lim)
    return fail(QMM_ERR_SHAPE, "x, qweight, zeros and scales must each be smaller than 4 GiB");
  return QMM_OK;
}

qmm_status check_product(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                         int group_size, const uint16_t* y, int max_m) {
  const qmm_status st = check_product_shape(M, K, N, bits, group_size, max_m);
  if (st != QMM_OK) return st;
  if (!x || !qweight || !zeros || !scales || !y) return fail(QMM_ERR_NULL, "a required pointer is NULL");
  if (bits == 3 && !qweight_lo) return fail(QMM_ERR_NULL, "qweight_lo (1-bit plane) is NULL for 3-bit codes");
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(zeros) || !aligned16(scales) || !aligned16(y) ||
      (bits == 3 && !aligned16(qweight_lo)))
    return fail(QMM_ERR_ALIGN, "x, qweight, qweight_lo, zeros, scales and y must be 16-byte aligned");
  if (!aligned(bias, 2)) return fail(QMM_ERR_ALIGN, "bias must be 2-byte aligned");
  return QMM_OK;
}

// Planes in the strip-major layout hold N rounded up to a multiple of 16
// columns; each must stay below 4 GiB, as the kernels' byte offsets are 32-bit.
qmm_status check_strips_planes(int K, int N, int bits) {
  const unsigned long long cols = (unsigned long long)qmm::plane_cols(N, 1);
  if ((unsigned long long)K * cols * (bits == 3 ? 2 : bits) / 8 >= (1ull << 32))
    return fail(QMM_ERR_SHAPE, "qweight in 16-column strips must be smaller than 4 GiB");
  return QMM_OK;
}

qmm_status check_flags(unsigned flags) {
  if (flags & ~(unsigned)(QMM_BF16 | QMM_STRIPS)) return fail(QMM_ERR_FLAGS, "flags=0x%x: unknown bits", flags);
  return QMM_OK;
}

qmm_status check_strips_call(const void* in, int rows, int N, const void* out) {
  if (rows < 1 || N < 1) return fail(QMM_ERR_SHAPE, "rows=%d and N=%d must be >= 1", rows, N);
  if ((unsigned long long)rows * (unsigned long long)qmm::plane_cols(N, 1) * 4 >= (1ull << 32))
    return fail(QMM_ERR_SHAPE, "a plane of %d rows and %d columns in strips must be smaller than 4 GiB", rows, N);
  if (!in || !out) return fail(QMM_ERR_NULL, "the input and output planes must not be NULL");
  if (!aligned(in, 4) || !aligned(out, 4)) return fail(QMM_ERR_ALIGN, "the planes must be 4-byte aligned");
  return QMM_OK;
}

qmm_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

qmm_status dequant_impl(const int32_t* qweight, const int32_t* qweight_lo, const uint16_t* zeros,
                       const uint16_t* scales, int K, int N, int bits, int group_size, uint16_t* w,
                       bool bf16, hipStream_t stream) {
  qmm_status st = check_packing(K, N, bits, qweight, qweight_lo);
  if (st != QMM_OK) return st;
  if (K % 32) return fail(QMM_ERR_SHAPE, "K=%d must be a multiple of 32", K);
  st = check_group(K, group_size);
  if (st != QMM_OK) return st;
  if (!zeros || !scales || !w) return fail(QMM_ERR_NULL, "zeros, scales and w must not be NULL");
  if (!aligned(qweight, 4) || (bits == 3 && !aligned(qweight_lo, 4)) || !aligned(zeros, 2) || !aligned(scales, 2) ||
      !aligned(w, 2))
    return fail(QMM_ERR_ALIGN, "qweight and qweight_lo must be 4-byte aligned, zeros, scales and w 2-byte aligned");
  return from_hip(qmm::launch_dequant(reinterpret_cast<const uint32_t*>(qweight),
                                      reinterpret_cast<const uint32_t*>(qweight_lo), zeros, scales, K, N, bits,
                                      group_size, w, bf16, stream),
                  "qmm_dequant launch");
}

qmm_status gemv_impl(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                    int group_size, uint16_t* y, void* workspace, size_t workspace_bytes, bool bf16,
                    bool strips, hipStream_t stream) {
  qmm_status st = check_product(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, 16);
  if (st != QMM_OK) return st;
  if (strips && (st = check_strips_planes(K, N, bits)) != QMM_OK) return st;
  if (N > qmm::kGemvMaxN) return fail(QMM_ERR_SHAPE, "N=%d exceeds the decode product's limit of %d", N, qmm::kGemvMaxN);
  const qmm::GemvPlan plan = qmm::gemv_plan(M, K, N, bits, group_size, qmm::device_topology());
  if (!plan.valid)
    return fail(QMM_ERR_SHAPE, "M=%d, K=%d, group_size=%d exceed the decode product's staging limits; use qmm_gemm",
                M, K, group_size);
  if (plan.workspace_bytes > 0) {
    if (!workspace) return fail(QMM_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", plan.workspace_bytes);
    if (workspace_bytes < plan.workspace_bytes)
      return fail(QMM_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, plan.workspace_bytes);
    if (!aligned16(workspace)) return fail(QMM_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  return from_hip(qmm::launch_gemv(plan, x, M, K, reinterpret_cast<const uint32_t*>(qweight),
                                   reinterpret_cast<const uint32_t*>(qweight_lo), zeros, scales, bias, N, bits,
                                   group_size, y, workspace, bf16, strips, stream),
                  "qmm_gemv launch");
}

// ---- the decode product without a caller workspace ----------------------------
// Device memory of a fixed size in the library's own code object, for callers
// that cannot allocate. It holds what a workspace holds: the arrival counters
// (zero when the code object is loaded, as every static device variable, and
// left at zero by each call) and the split-K partial sums. Every GPU has its
// own copy; in host code the array's name is only a stand-in for it, so its
// device address is looked up once per device and used everywhere instead.
constexpr size_t kScratchBytes = size_t(4) << 20;  // 4 MiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch, looked up on the first
// call on that device (with that device current).
qmm_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QMM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(QMM_ERR_HIP, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(QMM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QMM_OK;
}

qmm_status gemv_noalloc_impl(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                             const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                             int group_size, uint16_t* y, hipStream_t stream) {
  qmm_status st = check_product(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, 16);
  if (st != QMM_OK) return st;
  if (N > qmm::kGemvMaxN) return fail(QMM_ERR_SHAPE, "N=%d exceeds the decode product's limit of %d", N, qmm::kGemvMaxN);
  const qmm::GemvPlan plan = qmm::gemv_plan(M, K, N, bits, group_size, qmm::device_topology());
  if (!plan.valid)
    return fail(QMM_ERR_SHAPE, "M=%d, K=%d, group_size=%d exceed the decode product's staging limits; use qmm_gemm",
                M, K, group_size);
  if (plan.workspace_bytes > kScratchBytes)
    return fail(QMM_ERR_WORKSPACE, "this shape needs %zu bytes of scratch, more than the %zu the library holds; "
                "use qmm_gemv with a workspace", plan.workspace_bytes, kScratchBytes);
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    st = scratch_for_current_device(&ws);
    if (st != QMM_OK) return st;
  }
  return from_hip(qmm::launch_gemv(plan, x, M, K, reinterpret_cast<const uint32_t*>(qweight),
                                   reinterpret_cast<const uint32_t*>(qweight_lo), zeros, scales, bias, N, bits,
                                   group_size, y, ws, false, false, stream),
                  "qmm_gemv_noalloc launch");
}

qmm_status gemm_impl(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                    int group_size, uint16_t* y, bool bf16, bool strips, hipStream_t stream) {
  qmm_status st = check_product(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, 1 << 30);
  if (st != QMM_OK) return st;
  if (strips && (st = check_strips_planes(K, N, bits)) != QMM_OK) return st;
  return from_hip(qmm::launch_gemm(x, M, K, reinterpret_cast<const uint32_t*>(qweight),
                                   reinterpret_cast<const uint32_t*>(qweight_lo), zeros, scales, bias, N, bits,
                                   group_size, y, bf16, strips, qmm::device_topology(), stream),
                  "qmm_gemm launch");
}

}  // namespace

extern "C" {

int qmm_abi_version(void) { return QMM_ABI_VERSION; }

const char* qmm_status_string(int status) {
  switch (status) {
    case QMM_OK: return "QMM_OK";
    case QMM_ERR_NULL: return "QMM_ERR_NULL";
    case QMM_ERR_BITS: return "QMM_ERR_BITS";
    case QMM_ERR_SHAPE: return "QMM_ERR_SHAPE";
    case QMM_ERR_GROUP: return "QMM_ERR_GROUP";
    case QMM_ERR_ALIGN: return "QMM_ERR_ALIGN";
    case QMM_ERR_WORKSPACE: return "QMM_ERR_WORKSPACE";
    case QMM_ERR_HIP: return "QMM_ERR_HIP";
    case QMM_ERR_FLAGS: return "QMM_ERR_FLAGS";
    default: return "QMM_ERR_UNKNOWN";
  }
}

const char* qmm_last_error(void) { return g_last_error; }

qmm_status qmm_pack(const uint8_t* codes, int K, int N, int bits, int32_t* qweight, int32_t* qweight_lo,
                    int32_t* bad_count, hipStream_t stream) {
  qmm_status st = check_packing(K, N, bits, qweight, qweight_lo);
  if (st != QMM_OK) return st;
  if (!codes) return fail(QMM_ERR_NULL, "codes is NULL");
  return from_hip(qmm::launch_pack(codes, K, N, bits, reinterpret_cast<uint32_t*>(qweight),
                                   reinterpret_cast<uint32_t*>(qweight_lo), bad_count, stream),
                  "qmm_pack launch");
}

qmm_status qmm_unpack(const int32_t* qweight, const int32_t* qweight_lo, int K, int N, int bits, uint8_t* codes,
                      hipStream_t stream) {
  qmm_status st = check_packing(K, N, bits, qweight, qweight_lo);
  if (st != QMM_OK) return st;
  if (!codes) return fail(QMM_ERR_NULL, "codes is NULL");
  return from_hip(qmm::launch_unpack(reinterpret_cast<const uint32_t*>(qweight),
                                     reinterpret_cast<const uint32_t*>(qweight_lo), K, N, bits, codes, stream),
                  "qmm_unpack launch");
}

size_t qmm_workspace_bytes(int M, int K, int N, int bits, int group_size) {
  // A size query reports nothing: the last error message stays as it was.
  char saved[sizeof g_last_error];
  memcpy(saved, g_last_error, sizeof saved);
  const qmm_status st = check_product_shape(M, K, N, bits, group_size, 16);
  memcpy(g_last_error, saved, sizeof saved);
  if (st != QMM_OK || N > qmm::kGemvMaxN) return 0;
  return qmm::gemv_plan(M, K, N, bits, group_size, qmm::device_topology()).workspace_bytes;
}

qmm_status qmm_gemv_plan_info(int M, int K, int N, int bits, int group_size, int32_t* info, int n) {
  const qmm_status st = check_product_shape(M, K, N, bits, group_size, 16);
  if (st != QMM_OK) return st;
  if (N > qmm::kGemvMaxN) return fail(QMM_ERR_SHAPE, "N=%d exceeds the decode product's limit of %d", N, qmm::kGemvMaxN);
  if (n > 0 && !info) return fail(QMM_ERR_NULL, "info is NULL");
  const qmm::DeviceTopo topo = qmm::device_topology();
  const qmm::GemvPlan p = qmm::gemv_plan(M, K, N, bits, group_size, topo);
  if (!p.valid)
    return fail(QMM_ERR_SHAPE, "M=%d, K=%d, group_size=%d exceed the decode product's staging limits", M, K,
                group_size);
  const int32_t v[10] = {p.kind, p.vec, p.waves, p.nstrips, p.ksplit,
                         p.kind == 1 ? p.upw : p.units_per_block, p.kind == 1 ? p.gpw : 0, p.xcds, topo.cus,
                         p.kind == 1 && p.one_xcd > 1 ? 1 : 0};
  for (int i = 0; i < n && i < 10; ++i) info[i] = v[i];
  return ok();
}

qmm_status qmm_gemm_plan_info(int M, int K, int N, int bits, int group_size, int32_t* info, int n) {
  const qmm_status st = check_product_shape(M, K, N, bits, group_size, 1 << 30);
  if (st != QMM_OK) return st;
  if (n > 0 && !info) return fail(QMM_ERR_NULL, "info is NULL");
  const qmm::GemmPlan p = qmm::gemm_plan(M, K, N, qmm::device_topology());
  const int32_t v[7] = {p.bm, p.bn, p.kgroups, p.waves, (int32_t)(p.blocks < INT32_MAX ? p.blocks : INT32_MAX),
                        p.xcds, p.cus};
  for (int i = 0; i < n && i < 7; ++i) info[i] = v[i];
  return ok();
}

qmm_status qmm_dequant(const int32_t* qweight, const int32_t* qweight_lo, const uint16_t* zeros,
                       const uint16_t* scales, int K, int N, int bits, int group_size, uint16_t* w,
                       hipStream_t stream) {
  return dequant_impl(qweight, qweight_lo, zeros, scales, K, N, bits, group_size, w, false, stream);
}

qmm_status qmm_dequant_bf16(const int32_t* qweight, const int32_t* qweight_lo, const uint16_t* zeros,
                            const uint16_t* scales, int K, int N, int bits, int group_size, uint16_t* w,
                            hipStream_t stream) {
  return dequant_impl(qweight, qweight_lo, zeros, scales, K, N, bits, group_size, w, true, stream);
}

qmm_status qmm_gemv(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                    int group_size, uint16_t* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gemv_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, workspace,
                   workspace_bytes, false, false, stream);
}

qmm_status qmm_gemv_bf16(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                         int group_size, uint16_t* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gemv_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, workspace,
                   workspace_bytes, true, false, stream);
}

qmm_status qmm_gemv_noalloc(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                            const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                            int group_size, uint16_t* y, hipStream_t stream) {
  return gemv_noalloc_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, stream);
}

qmm_status qmm_gemm(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                    int group_size, uint16_t* y, hipStream_t stream) {
  return gemm_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, false, false, stream);
}

qmm_status qmm_gemm_bf16(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                         int group_size, uint16_t* y, hipStream_t stream) {
  return gemm_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, true, false, stream);
}

qmm_status qmm_gemv_ex(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                       const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                       int group_size, unsigned flags, uint16_t* y, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  const qmm_status st = check_flags(flags);
  if (st != QMM_OK) return st;
  return gemv_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, workspace,
                   workspace_bytes, (flags & QMM_BF16) != 0, (flags & QMM_STRIPS) != 0, stream);
}

qmm_status qmm_gemm_ex(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                       const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                       int group_size, unsigned flags, uint16_t* y, hipStream_t stream) {
  const qmm_status st = check_flags(flags);
  if (st != QMM_OK) return st;
  return gemm_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y,
                   (flags & QMM_BF16) != 0, (flags & QMM_STRIPS) != 0, stream);
}

size_t qmm_strips_bytes(int rows, int N) {
  if (rows < 1 || N < 1) return 0;
  const unsigned long long b = (unsigned long long)rows * (unsigned long long)qmm::plane_cols(N, 1) * 4;
  return b >= (1ull << 32) ? 0 : (size_t)b;
}

qmm_status qmm_to_strips(const int32_t* words, int rows, int N, int32_t* strips, hipStream_t stream) {
  const qmm_status st = check_strips_call(words, rows, N, strips);
  if (st != QMM_OK) return st;
  return from_hip(qmm::launch_to_strips(reinterpret_cast<const uint32_t*>(words), rows, N,
                                        reinterpret_cast<uint32_t*>(strips), stream),
                  "qmm_to_strips launch");
}

qmm_status qmm_from_strips(const int32_t* strips, int rows, int N, int32_t* words, hipStream_t stream) {
  const qmm_status st = check_strips_call(strips, rows, N, words);
  if (st != QMM_OK) return st;
  return from_hip(qmm::launch_from_strips(reinterpret_cast<const uint32_t*>(strips), rows, N,
                                          reinterpret_cast<uint32_t*>(words), stream),
                  "qmm_from_strips launch");
}

}  // extern "C"
