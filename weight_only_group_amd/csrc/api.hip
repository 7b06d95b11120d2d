// C ABI: argument validation, error reporting and dispatch to the kernels.
// Every check runs on the host before anything is enqueued; no HIP call is
// made for an invalid request.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/qmm.h"
#include "common.h"
#include "gptq.h"

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

qmm_status check_product(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                         int group_size, const uint16_t* y, int max_m) {
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
  if (!x || !qweight || !zeros || !scales || !y) return fail(QMM_ERR_NULL, "a required pointer is NULL");
  if (bits == 3 && !qweight_lo) return fail(QMM_ERR_NULL, "qweight_lo (1-bit plane) is NULL for 3-bit codes");
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(zeros) || !aligned16(scales) || !aligned16(y) ||
      (bits == 3 && !aligned16(qweight_lo)))
    return fail(QMM_ERR_ALIGN, "x, qweight, qweight_lo, zeros, scales and y must be 16-byte aligned");
  if (!aligned(bias, 2)) return fail(QMM_ERR_ALIGN, "bias must be 2-byte aligned");
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
                    hipStream_t stream) {
  qmm_status st = check_product(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, 16);
  if (st != QMM_OK) return st;
  if (N > qmm::kGemvMaxN) return fail(QMM_ERR_SHAPE, "N=%d exceeds the decode product's limit of %d", N, qmm::kGemvMaxN);
  const qmm::GemvPlan plan = qmm::gemv_plan(M, K, N, bits, group_size);
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
                                   group_size, y, workspace, bf16, stream),
                  "qmm_gemv launch");
}

qmm_status unpack_qzeros_impl(const int32_t* qzeros, int G, int N, int bits, uint16_t* zeros, bool bf16,
                              hipStream_t stream) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(QMM_ERR_BITS, "bits=%d: packed zero points come in 2, 3, 4 or 8 bits", bits);
  if (G < 1 || N < 1) return fail(QMM_ERR_SHAPE, "G=%d and N=%d must be >= 1", G, N);
  if ((unsigned long long)G * N * 2 >= (1ull << 32)) return fail(QMM_ERR_SHAPE, "zeros must be smaller than 4 GiB");
  if (!qzeros || !zeros) return fail(QMM_ERR_NULL, "qzeros and zeros must not be NULL");
  if (!aligned(qzeros, 4) || !aligned(zeros, 2))
    return fail(QMM_ERR_ALIGN, "qzeros must be 4-byte aligned and zeros 2-byte aligned");
  return from_hip(qmm::launch_unpack_qzeros(reinterpret_cast<const uint32_t*>(qzeros), G, N, bits, zeros, bf16,
                                            stream),
                  "qmm_unpack_qzeros launch");
}

qmm_status gemm_impl(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                    int group_size, uint16_t* y, bool bf16, hipStream_t stream) {
  qmm_status st = check_product(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, 1 << 30);
  if (st != QMM_OK) return st;
  return from_hip(qmm::launch_gemm(x, M, K, reinterpret_cast<const uint32_t*>(qweight),
                                   reinterpret_cast<const uint32_t*>(qweight_lo), zeros, scales, bias, N, bits,
                                   group_size, y, bf16, stream),
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
  if (!bits_ok(bits) || M < 1 || M > 16 || K < 32 || K % 32 || N < 8 || N % 8 || N > qmm::kGemvMaxN) return 0;
  if (group_size != -1 && (group_size <= 0 || group_size % 32 || K % group_size)) return 0;
  return qmm::gemv_plan(M, K, N, bits, group_size).workspace_bytes;
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
                   workspace_bytes, false, stream);
}

qmm_status qmm_gemv_bf16(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                         int group_size, uint16_t* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gemv_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, workspace,
                   workspace_bytes, true, stream);
}

qmm_status qmm_gemm(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                    int group_size, uint16_t* y, hipStream_t stream) {
  return gemm_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, false, stream);
}

qmm_status qmm_gemm_bf16(const uint16_t* x, int M, int K, const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                         int group_size, uint16_t* y, hipStream_t stream) {
  return gemm_impl(x, M, K, qweight, qweight_lo, zeros, scales, bias, N, bits, group_size, y, true, stream);
}

qmm_status qmm_unpack_qzeros(const int32_t* qzeros, int G, int N, int bits, uint16_t* zeros, hipStream_t stream) {
  return unpack_qzeros_impl(qzeros, G, N, bits, zeros, false, stream);
}

qmm_status qmm_unpack_qzeros_bf16(const int32_t* qzeros, int G, int N, int bits, uint16_t* zeros,
                                  hipStream_t stream) {
  return unpack_qzeros_impl(qzeros, G, N, bits, zeros, true, stream);
}

qmm_status qmm_repack_3bit10(const int32_t* qweight10, int K, int N, int32_t* qweight, int32_t* qweight_lo,
                             hipStream_t stream) {
  if (K < 32 || K % 32) return fail(QMM_ERR_SHAPE, "K=%d must be a positive multiple of 32", K);
  if (N < 1) return fail(QMM_ERR_SHAPE, "N=%d must be >= 1", N);
  if ((unsigned long long)((K + 9) / 10) * N * 4 >= (1ull << 32))
    return fail(QMM_ERR_SHAPE, "qweight10 must be smaller than 4 GiB");
  if (!qweight10 || !qweight || !qweight_lo) return fail(QMM_ERR_NULL, "qweight10, qweight and qweight_lo must not be NULL");
  if (!aligned(qweight10, 4) || !aligned(qweight, 4) || !aligned(qweight_lo, 4))
    return fail(QMM_ERR_ALIGN, "qweight10, qweight and qweight_lo must be 4-byte aligned");
  return from_hip(qmm::launch_repack_3bit10(reinterpret_cast<const uint32_t*>(qweight10), K, N,
                                            reinterpret_cast<uint32_t*>(qweight),
                                            reinterpret_cast<uint32_t*>(qweight_lo), stream),
                  "qmm_repack_3bit10 launch");
}

}  // extern "C"
