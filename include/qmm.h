/*
 * qmm.h -- C ABI of the weight-only, group-wise asymmetric integer quantized
 * matmul for AMD Instinct MI355X (gfx950).
 *
 *   y[m, n] = sum_k x[m, k] * scale[g, n] * (q[k, n] - zero[g, n]),  g = k / group_size
 *
 * The operation and its arguments follow the functional statement of the
 * problem in the GPTQModel-Compatible Triton Kernel README ("API Reference":
 * gptqmodel_quantized_matmul(x, qweight, qzeros, scales, bits, group_size),
 * output = x @ dequantize(qweight); "Dequantization Formula"; "Group
 * Quantization": group_size -1 is one scale/zero per output channel). The
 * weight layout is the K-major packing of dashq_kernel.py (module docstring,
 * _pack_kmajor / _unpack_kmajor): a (K / eps, N) int32 array, eps = 32 / bits,
 * code k of column n in word k / eps at bit offset (k % eps) * bits; 3-bit
 * codes are a 2-bit plane of q >> 1 plus a 1-bit plane of q & 1. Widths 1, 2,
 * 3, 4 and 8 are supported (dashq_kernel.py, SUPPORTED_NBITS). An optional
 * bias row is added to the fp32 result before its rounding to fp16
 * (dashq_kernel.py, TritonQuantLinear: the accumulator starts from the bias).
 * The _bf16 entry points take and return bfloat16 data instead of fp16 (x,
 * zeros, scales, bias, y, w as bf16 bit patterns; dashq_kernel.py keeps
 * scales and zeros in the module's output dtype and returns the product in
 * the activations' dtype); everything else is the same.
 *
 * Conventions for every entry point:
 *  - Pointers to arrays are DEVICE pointers (memory of the current HIP
 *    device); all arrays are dense and row-major; fp16 values are passed as
 *    uint16_t IEEE binary16 bit patterns; int32 words are read as unsigned
 *    32-bit patterns (logical shifts).
 *  - The caller owns every buffer. The library allocates nothing per call and
 *    keeps no pointer after returning.
 *  - Arguments are validated on the host before anything is enqueued. On any
 *    error nothing is enqueued, outputs are untouched, the status says why and
 *    qmm_last_error() holds a message (per thread).
 *  - QMM_OK means the work was enqueued on `stream` (0 = the null stream);
 *    completion is observed by synchronising that stream. A kernel launch
 *    error is reported as QMM_ERR_HIP.
 *  - Calls are reentrant; calls that share a workspace must not overlap.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMM_ABI_VERSION 4

typedef enum qmm_status {
  QMM_OK = 0,
  QMM_ERR_NULL = 1,      /* a required pointer is NULL                              */
  QMM_ERR_BITS = 2,      /* bits not in {1, 2, 3, 4, 8}                             */
  QMM_ERR_SHAPE = 3,     /* M, K or N out of range or not a required multiple      */
  QMM_ERR_GROUP = 4,     /* group_size neither -1 nor a positive multiple of 32 dividing K */
  QMM_ERR_ALIGN = 5,     /* a pointer is not aligned as its argument requires        */
  QMM_ERR_WORKSPACE = 6, /* workspace missing or smaller than qmm_workspace_bytes() */
  QMM_ERR_HIP = 7        /* the HIP runtime reported an error                       */
} qmm_status;

/* QMM_ABI_VERSION of the built library. */
int qmm_abi_version(void);

/* Static text naming a status code ("QMM_OK", ...); never NULL. */
const char* qmm_status_string(int status);

/* Message of the last failed call on this thread ("" if none); valid until
 * the next call on this thread. */
const char* qmm_last_error(void);

/*
 * qmm_pack -- codes (K, N) uint8, row-major -> K-major packed words.
 * Defined by dashq_kernel.py, _pack_kmajor and TritonQuantLinear.__init__
 * (3-bit planes).
 *   bits 1, 2, 4, 8: qweight (K / eps, N) int32, eps = 32 / bits; qweight_lo unused (may be NULL).
 *   bits 3:       qweight = 2-bit plane of q >> 1, (K / 16, N); qweight_lo = 1-bit
 *                 plane of q & 1, (K / 32, N).
 * Requirements: K % eps == 0 (K % 32 == 0 for 3 bits), N >= 1, K >= 1.
 * Codes wider than `bits` are masked to their low `bits` bits. If bad_count is
 * not NULL it points to one device int32 that the caller has zeroed; the
 * number of such codes is added to it.
 */
qmm_status qmm_pack(const uint8_t* codes, int K, int N, int bits,
                    int32_t* qweight, int32_t* qweight_lo, int32_t* bad_count,
                    hipStream_t stream);

/*
 * qmm_unpack -- inverse of qmm_pack: packed words -> codes (K, N) uint8.
 * Defined by dashq_kernel.py, _unpack_kmajor and dequantize_weight
 * (q = (plane2 << 1) | plane1 for 3 bits). Same shapes and requirements as
 * qmm_pack; every output code is < 2**bits.
 */
qmm_status qmm_unpack(const int32_t* qweight, const int32_t* qweight_lo, int K, int N, int bits,
                      uint8_t* codes, hipStream_t stream);

/*
 * qmm_dequant -- the dequantized weight as fp16, K-major (K, N) row-major:
 *   w[k, n] = fp16(scale[g, n] * (q[k, n] - zero[g, n])),  g = k / group_size
 * dashq_kernel.py, TritonQuantLinear.dequantize_weight (the step its batched
 * path runs before a dense product). The exact product is rounded once to
 * fp16, nearest even.
 *   qweight, qweight_lo   packed words as written by qmm_pack (qweight_lo only for 3 bits)
 *   zeros, scales         (G, N) fp16, G = K / group_size, or 1 if group_size == -1
 *   w                     (K, N) fp16 output
 * Requirements: K % 32 == 0, N >= 1, group_size == -1 or (group_size % 32 == 0
 * and K % group_size == 0). No alignment beyond the element size is needed
 * (4 bytes for the packed words, 2 for zeros, scales and w; QMM_ERR_ALIGN).
 */
qmm_status qmm_dequant(const int32_t* qweight, const int32_t* qweight_lo,
                       const uint16_t* zeros, const uint16_t* scales,
                       int K, int N, int bits, int group_size,
                       uint16_t* w, hipStream_t stream);

/* qmm_dequant for bf16 scales and zero points; w is bf16, the exact product
 * rounded once to bf16, nearest even. */
qmm_status qmm_dequant_bf16(const int32_t* qweight, const int32_t* qweight_lo,
                            const uint16_t* zeros, const uint16_t* scales,
                            int K, int N, int bits, int group_size,
                            uint16_t* w, hipStream_t stream);

/*
 * qmm_workspace_bytes -- device workspace qmm_gemv needs for this problem
 * (0 if it needs none; also 0 for invalid arguments). The workspace holds a
 * fixed 128 KiB header of per-column-strip arrival counters followed by
 * split-K partial sums. It must be zero-filled once when allocated; qmm_gemv
 * leaves the counters at zero again when it completes, so the same workspace
 * can be reused call after call, for any shape it is large enough for.
 */
size_t qmm_workspace_bytes(int M, int K, int N, int bits, int group_size);

/*
 * qmm_gemv -- y = x @ dequantize(W) for small M (1 <= M <= 16), the decode
 * product. dashq_kernel.py, _dashq_gemv_kernel and TritonQuantLinear.forward
 * (single-token path); GPTQModel-Compatible Triton Kernel README, "API
 * Reference".
 *   x       (M, K) fp16
 *   qweight, qweight_lo   packed words as written by qmm_pack (qweight_lo only for 3 bits)
 *   zeros, scales         (G, N) fp16, G = K / group_size, or 1 if group_size == -1
 *   bias    (N,) fp16 or NULL; added to the fp32 result before rounding
 *   y       (M, N) fp16 output, fp32 accumulation, rounded to nearest even
 *   workspace, workspace_bytes   see qmm_workspace_bytes
 * Requirements: K % 32 == 0, N % 8 == 0, N <= 1048576, group_size == -1 or
 * (group_size % 32 == 0 and K % group_size == 0); x, qweight, qweight_lo,
 * zeros, scales, y and workspace 16-byte aligned, bias 2-byte aligned; x, each packed plane,
 * zeros and scales smaller than 4 GiB. Shapes whose activations or scales do
 * not fit the kernel's on-chip staging (M * K large, e.g. K > 32768 at
 * M = 16) are rejected with QMM_ERR_SHAPE; qmm_gemm takes them.
 * The summation order is fixed: two calls on the same inputs give the same bits.
 * One zero-filled workspace serves calls of any shape, as long as it is large
 * enough for each and calls sharing it do not overlap in time.
 */
qmm_status qmm_gemv(const uint16_t* x, int M, int K,
                    const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias,
                    int N, int bits, int group_size,
                    uint16_t* y, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* qmm_gemv with bf16 x, zeros, scales, bias and y (the same workspace). The
 * dequantized codes are formed in fp32 and rounded once to bf16 for the
 * matrix cores; accumulation stays fp32 and y is rounded to nearest even. */
qmm_status qmm_gemv_bf16(const uint16_t* x, int M, int K,
                         const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias,
                         int N, int bits, int group_size,
                         uint16_t* y, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * qmm_gemm -- the same product for any M >= 1, the prefill product: packed
 * tiles are dequantized to fp16 in LDS and multiplied on the matrix cores
 * with fp32 accumulation. dashq_kernel.py, TritonQuantLinear.forward (batched
 * path: dequantize, then a dense product); GPTQModel-Compatible Triton Kernel
 * README, overview (dequantization fused with the product).
 * Arguments and requirements as for qmm_gemv (bias included), without a
 * workspace and without the staging limit.
 */
qmm_status qmm_gemm(const uint16_t* x, int M, int K,
                    const int32_t* qweight, const int32_t* qweight_lo,
                    const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias,
                    int N, int bits, int group_size,
                    uint16_t* y, hipStream_t stream);

/* qmm_gemm with bf16 x, zeros, scales, bias and y (as qmm_gemv_bf16). */
qmm_status qmm_gemm_bf16(const uint16_t* x, int M, int K,
                         const int32_t* qweight, const int32_t* qweight_lo,
                         const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias,
                         int N, int bits, int group_size,
                         uint16_t* y, hipStream_t stream);

/*
 * GPTQModel-format inputs. GPTQModel-Compatible Triton Kernel README, "API
 * Reference" (qzeros: the packed quantized zero points) and "Quantization
 * Format" (int32 words of 16, 10, 8 or 4 values for 2, 3, 4 or 8 bits, the
 * 3-bit words padded). The README does not say where a value sits in its word
 * or along which axis the zero points are packed. Read here as: value i of a
 * word at bit offset i * bits, lowest first (3-bit words hold 10 values in
 * bits 0-29, bits 30-31 unused); weights packed along K, zero points along N;
 * the last word of a row or column partly filled; the stored zero point is
 * used as is (w = scale * (q - zero), "Dequantization Formula"). In this
 * reading 2-, 4- and 8-bit GPTQModel weight words are the K-major words the
 * products take; the two calls below convert the rest, once, at load time.
 */

/*
 * qmm_unpack_qzeros -- packed zero points -> (G, N) fp16 zero points.
 *   qzeros  (G, ceil(N / e)) int32, e = 16, 10, 8, 4 for bits 2, 3, 4, 8;
 *           zero point n of group g in word n / e of row g at bit offset
 *           (n % e) * bits
 *   zeros   (G, N) fp16 output: the integer zero points, exact
 * Requirements: bits in {2, 3, 4, 8} (QMM_ERR_BITS); G, N >= 1 (QMM_ERR_SHAPE);
 * qzeros 4-byte and zeros 2-byte aligned (QMM_ERR_ALIGN).
 */
qmm_status qmm_unpack_qzeros(const int32_t* qzeros, int G, int N, int bits,
                             uint16_t* zeros, hipStream_t stream);

/* qmm_unpack_qzeros writing bf16 zero points (exact: integers below 256). */
qmm_status qmm_unpack_qzeros_bf16(const int32_t* qzeros, int G, int N, int bits,
                                  uint16_t* zeros, hipStream_t stream);

/*
 * qmm_repack_3bit10 -- 3-bit GPTQModel weights, 10 codes per word packed
 * along K, -> the two planes of the 3-bit layout, as qmm_pack writes them.
 *   qweight10   (ceil(K / 10), N) int32; code k of column n in word k / 10 at
 *               bit offset 3 (k % 10); bits 30-31 and the slots past K ignored
 *   qweight     (K / 16, N) int32 output: the 2-bit plane of q >> 1
 *   qweight_lo  (K / 32, N) int32 output: the 1-bit plane of q & 1
 * Requirements: K a positive multiple of 32 (the planes' granularity) and
 * N >= 1 (QMM_ERR_SHAPE); every pointer 4-byte aligned (QMM_ERR_ALIGN).
 */
qmm_status qmm_repack_3bit10(const int32_t* qweight10, int K, int N,
                             int32_t* qweight, int32_t* qweight_lo, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
