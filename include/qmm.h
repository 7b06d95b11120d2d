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

#define QMM_ABI_VERSION 6

typedef enum qmm_status {
  QMM_OK = 0,
  QMM_ERR_NULL = 1,      /* a required pointer is NULL                              */
  QMM_ERR_BITS = 2,      /* bits not in {1, 2, 3, 4, 8}                             */
  QMM_ERR_SHAPE = 3,     /* M, K or N out of range or not a required multiple      */
  QMM_ERR_GROUP = 4,     /* group_size neither -1 nor a positive multiple of 32 dividing K */
  QMM_ERR_ALIGN = 5,     /* a pointer is not aligned as its argument requires        */
  QMM_ERR_WORKSPACE = 6, /* workspace missing or smaller than qmm_workspace_bytes() */
  QMM_ERR_HIP = 7,       /* the HIP runtime reported an error                       */
  QMM_ERR_FLAGS = 8      /* a flags argument has bits other than QMM_BF16 | QMM_STRIPS */
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
 * qmm_gemv_plan_info -- the launch plan qmm_gemv (and qmm_gemv_bf16,
 * qmm_gemv_noalloc) uses for this problem on the current device, for tests
 * and measurement. Host only: no work is enqueued. Writes min(n, 10) ints:
 *   info[0] kernel: 0 = blocks split along K (partial sums through the
 *           workspace when info[4] > 1), 1 = one block per column strip, each
 *           wave over its own K range
 *   info[1] adjacent columns per lane (1, 2 or 4); a wave covers 16 * info[1]
 *   info[2] waves per block
 *   info[3] blocks along N (column strips)
 *   info[4] blocks along K
 *   info[5] 32-row units of K per wave (kernel 1) or per block (kernel 0)
 *   info[6] groups per wave (kernel 1), else 0
 *   info[7] XCDs the strips are laid out for
 *   info[8] compute units of the device
 *   info[9] 1 if every strip runs on XCD 0 (kernel 1 with at most one strip
 *           per CU of an XCD and at most 1 MiB of weight words: the grid then
 *           holds one workgroup per strip on each XCD, and those dealt to the
 *           other XCDs return at once), else 0
 * Returns QMM_ERR_NULL for a NULL info with n > 0, QMM_ERR_SHAPE (etc.) for
 * arguments qmm_gemv would reject on shape alone, else QMM_OK.
 */
qmm_status qmm_gemv_plan_info(int M, int K, int N, int bits, int group_size, int32_t* info, int n);

/*
 * qmm_gemm_plan_info -- the block tiling qmm_gemm (and qmm_gemm_bf16) uses
 * for this problem on the current device, for tests and measurement. Host
 * only: no work is enqueued. Writes min(n, 7) ints:
 *   info[0] block tile rows     info[1] block tile columns
 *   info[2] groups of waves splitting a block's K range
 *   info[3] waves per block     info[4] blocks (capped at 2^31 - 1)
 *   info[5] XCDs the tiles are laid out for   info[6] compute units
 * Returns QMM_ERR_NULL for a NULL info with n > 0, QMM_ERR_SHAPE (etc.) for
 * arguments qmm_gemm would reject on shape alone, else QMM_OK.
 */
qmm_status qmm_gemm_plan_info(int M, int K, int N, int bits, int group_size, int32_t* info, int n);

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
 * qmm_gemv_noalloc -- qmm_gemv without a workspace argument, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation). It computes exactly what qmm_gemv
 * computes, with the same kernels and the same bits; where the plan needs
 * scratch memory (arrival counters and split-K partial sums), it uses a fixed
 * 4 MiB device array held by the library, one per GPU, for the life of the
 * process. The call itself allocates nothing.
 *   Arguments and requirements as for qmm_gemv, minus the workspace.
 *   Shapes needing more than 4 MiB of scratch (qmm_workspace_bytes() > 4 MiB:
 *   narrow N with a deep K split at large M) are refused with
 *   QMM_ERR_WORKSPACE; qmm_gemv with a workspace takes them.
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from several threads) race on it and
 * must be serialised by the caller. The arrival counters start at zero when
 * the library's code object is loaded and every call leaves them at zero.
 */
qmm_status qmm_gemv_noalloc(const uint16_t* x, int M, int K,
                            const int32_t* qweight, const int32_t* qweight_lo,
                            const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias,
                            int N, int bits, int group_size,
                            uint16_t* y, hipStream_t stream);

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
 * 16-column strip-major weights. The products read a plane of packed words
 * (rows x N int32: qweight, and qweight_lo for 3 bits) one column strip at a
 * time; the decode product gives each block 16 columns over all of K. In the
 * K-major layout above such a strip is a 64-byte piece of every word row;
 * qmm_to_strips reorders a plane once, at load time, so that every 16-column
 * strip is one contiguous run:
 *   word (r, n) of the plane at index ((n / 16) * rows + r) * 16 + n % 16,
 * a (ceil(N / 16), rows, 16) int32 array whose columns past N (in the last
 * strip, when N % 16 != 0) are zero. The words are the same (a permutation),
 * so the products return the same bits from either layout. Not a layout of
 * the pages: the packing they define (K-major words) stays the input format;
 * this is a storage order of the same words for the decode product's reads
 * (a strip is then streamed in order; 4096 x 4096 at 4 bits: ~8% less time).
 * qmm_gemv_ex / qmm_gemm_ex take it with QMM_STRIPS; qmm_dequant, qmm_unpack
 * and qmm_gemv_noalloc take the K-major layout only.
 */

/* Bytes of a plane of `rows` word rows and N columns in strip-major order:
 * rows * ceil(N / 16) * 16 * 4; 0 if rows < 1, N < 1 or the plane would
 * reach 4 GiB. */
size_t qmm_strips_bytes(int rows, int N);

/*
 * qmm_to_strips -- K-major plane -> strip-major plane.
 *   words   (rows, N) int32, e.g. qweight as written by qmm_pack (rows = K / eps;
 *           for 3 bits qweight has K / 16 rows and qweight_lo K / 32)
 *   strips  qmm_strips_bytes(rows, N) bytes, written completely
 * qmm_from_strips is the inverse (the padding columns are dropped).
 * Requirements: rows, N >= 1 and the strip-major plane below 4 GiB
 * (QMM_ERR_SHAPE); both pointers non-NULL (QMM_ERR_NULL) and 4-byte aligned
 * (QMM_ERR_ALIGN); the two planes must not overlap.
 */
qmm_status qmm_to_strips(const int32_t* words, int rows, int N, int32_t* strips, hipStream_t stream);
qmm_status qmm_from_strips(const int32_t* strips, int rows, int N, int32_t* words, hipStream_t stream);

/* Flags of the _ex products. */
#define QMM_BF16 1u   /* x, zeros, scales, bias and y are bf16 (as the _bf16 entry points) */
#define QMM_STRIPS 2u /* qweight and qweight_lo are in the strip-major layout (qmm_to_strips) */

/*
 * qmm_gemv_ex, qmm_gemm_ex -- qmm_gemv and qmm_gemm with a flags argument
 * (QMM_BF16, QMM_STRIPS, or both; other bits: QMM_ERR_FLAGS). With flags 0
 * they are qmm_gemv and qmm_gemm, with QMM_BF16 qmm_gemv_bf16 and
 * qmm_gemm_bf16. With QMM_STRIPS each packed plane is read in the
 * strip-major layout, which must hold below 4 GiB (QMM_ERR_SHAPE); every
 * other argument, requirement and result is as for the K-major call, and the
 * workspace is the same (qmm_workspace_bytes).
 */
qmm_status qmm_gemv_ex(const uint16_t* x, int M, int K,
                       const int32_t* qweight, const int32_t* qweight_lo,
                       const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias,
                       int N, int bits, int group_size, unsigned flags,
                       uint16_t* y, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);
qmm_status qmm_gemm_ex(const uint16_t* x, int M, int K,
                       const int32_t* qweight, const int32_t* qweight_lo,
                       const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias,
                       int N, int bits, int group_size, unsigned flags,
                       uint16_t* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
