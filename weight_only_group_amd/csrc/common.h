// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Two fp16 1024.0 values. OR-ing a code q < 1024 into the low mantissa bits of
// a half gives exactly 1024 + q, so one integer op turns two codes into two
// halves; subtracting 1024 (+ the zero point) afterwards is exact.
constexpr uint32_t kMagic1024x2 = 0x64006400u;
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int cmin(int a, int b) { return a < b ? a : b; }

__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(f16, b);
}

// 16-bit floating-point data is stored as bit patterns: IEEE binary16 (BF
// false) or bfloat16 (BF true, the upper half of a binary32).
template <bool BF>
__device__ __forceinline__ float bits_to_float(uint16_t b) {
  if constexpr (BF) return __builtin_bit_cast(float, (uint32_t)b << 16);
  else return (float)__builtin_bit_cast(f16, b);
}
// Rounded to nearest, ties to even.
template <bool BF>
__device__ __forceinline__ uint16_t float_to_bits(float v) {
  if constexpr (BF) return __builtin_bit_cast(uint16_t, (bf16)v);
  else return __builtin_bit_cast(uint16_t, (f16)v);
}
// Two floats as a bf16 pair (element 0 in the low half), each rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2{(bf16)lo, (bf16)hi});
}

// Rows of the weight per group: group_size, or K for group_size == -1.
inline int group_rows(int K, int group_size) { return group_size == -1 ? K : group_size; }

// ---- device topology ----------------------------------------------------------
// Compute units and XCDs (each XCD with its own L2) of the current device, read
// once per device; the MI355X values (256, 8) when no device can be queried.
struct DeviceTopo {
  int cus;
  int xcds;
};
DeviceTopo device_topology();

// ---- weight layouts ----------------------------------------------------------
// A plane of packed words (rows x N int32) is read in one of two layouts:
// K-major (word (r, n) at r * N + n, the packing of the products' inputs)
// or 16-column strip-major (word (r, n) at ((n / 16) * rows + r) * 16 +
// n % 16: every 16-column strip stored whole, row after row, the columns past
// N of the last strip padded). In both, word (r, n) sits at
// plane_col(n) + r * row stride.
constexpr int kStripCols = 16;
__host__ __device__ __forceinline__ int plane_row_stride(int N, int strips) { return strips ? kStripCols : N; }
__host__ __device__ __forceinline__ long long plane_cols(int N, int strips) {  // words per row as stored
  return strips ? ((long long)N + kStripCols - 1) / kStripCols * kStripCols : (long long)N;
}
__host__ __device__ __forceinline__ uint32_t plane_col(int n, int rows, int strips) {
  return strips ? (uint32_t)(n >> 4) * (uint32_t)rows * (uint32_t)kStripCols + (uint32_t)(n & 15) : (uint32_t)n;
}

// ---- decode GEMV (small M) ----------------------------------------------
// The workspace header has one arrival counter per column strip. Strips are
// 32 or 64 columns wide whenever there are more than 256 of them, so this
// covers every N up to the limit.
constexpr int kGemvMaxN = 1 << 20;
constexpr int kGemvMaxStrips = kGemvMaxN / 32;
struct GemvPlan {
  int kind;         // 0: blocks split K, waves sum through LDS, split-K hand-off; 1: wave kernel
  int vec;          // adjacent columns per lane (1, 2 or 4); a wave covers 16 * vec columns
  int waves;        // waves per block (4, 8 or 16), each taking a slice of the block's K range
  int strip_cols;   // columns per block
  int nstrips;      // blocks along N
  int ksplit;       // blocks along K
  int units_per_block;  // 32-row units of K per block
  int upg;          // 32-row units per group
  int upg_log2;     // log2(upg) if upg is a power of two, else -1
  int ubp_log2;     // log2 of the activation slots staged per row and lane group
  int gp_log2;      // log2 of the rows of scales / zero points staged per block
  int upw;          // wave kernel: 32-row units per wave (K / 32 = waves * upw)
  int gl;           // wave kernel: log2 of the units per group (30: one group)
  int gpw;          // wave kernel: groups per wave (1, 2 or 4)
  int xcds;         // XCDs of the device
  int one_xcd;      // wave kernel: strips all on XCD 0 (the grid holds xcds blocks per strip)
  size_t counters_bytes;  // arrival counters (one per strip), padded
  size_t workspace_bytes; // counters + split-K partial sums
  int valid;        // 0: the shape does not fit the decode product's staging limits
};
GemvPlan gemv_plan(int M, int K, int N, int bits, int group_size, DeviceTopo topo);
// bf16: x, zeros, scales, bias and y hold bfloat16 instead of fp16 bit patterns.
hipError_t launch_gemv(const GemvPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                       const uint32_t* qlo, const uint16_t* zeros, const uint16_t* scales,
                       const uint16_t* bias, int N, int bits, int group_size, uint16_t* y,
                       void* workspace, bool bf16, bool strips, hipStream_t stream);

// ---- prefill GEMM ---------------------------------------------------------
struct GemmPlan {
  int tile;       // block shape: 0 = 256 x 256, 1 = 128 x 128 (2 K groups), 2 / 3 = 64 x 64 (6 / 4 K groups)
  int bm, bn;     // block tile rows and columns
  int kgroups;    // groups of waves splitting a block's K range
  int waves;      // waves per block
  long long blocks;
  int xcds, cus;
};
GemmPlan gemm_plan(int M, int K, int N, DeviceTopo topo);
hipError_t launch_gemm(const uint16_t* x, int M, int K, const uint32_t* qw, const uint32_t* qlo,
                       const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N,
                       int bits, int group_size, uint16_t* y, bool bf16, bool strips, DeviceTopo topo,
                       hipStream_t stream);

// ---- strip-major re-layout (load time) ----------------------------------------
hipError_t launch_to_strips(const uint32_t* words, int rows, int N, uint32_t* strips, hipStream_t stream);
hipError_t launch_from_strips(const uint32_t* strips, int rows, int N, uint32_t* words, hipStream_t stream);

// ---- dequantize to fp16 -------------------------------------------------------
hipError_t launch_dequant(const uint32_t* qw, const uint32_t* qlo, const uint16_t* zeros,
                          const uint16_t* scales, int K, int N, int bits, int group_size, uint16_t* w,
                          bool bf16, hipStream_t stream);

// ---- pack / unpack ----------------------------------------------------------
hipError_t launch_pack(const uint8_t* codes, int K, int N, int bits, uint32_t* qw, uint32_t* qlo,
                       int32_t* bad_count, hipStream_t stream);
hipError_t launch_unpack(const uint32_t* qw, const uint32_t* qlo, int K, int N, int bits,
                         uint8_t* codes, hipStream_t stream);

}  // namespace qmm
