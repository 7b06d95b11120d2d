// The dequantized weight as fp16, K-major (K, N):
//   w[k, n] = fp16(scale[g, n] * (q[k, n] - zero[g, n])),  g = k / group_size
// (dashq_kernel.py, TritonQuantLinear.dequantize_weight: the (in_features,
// out_features) weight rebuilt from the packed codes, the group's zero point
// and its scale). The product is formed in fp64, where it is exact (the code
// difference and the scale are fp16 values; the product has at most 30
// significant bits), and rounded once to fp16, nearest even.
//
// One thread per 32-row chunk of one column: it reads the chunk's packed words
// (one word per bit of width; for 3-bit codes two words of the 2-bit plane and
// one of the 1-bit plane), the chunk's zero point and scale once (32 divides
// the group size), and writes 32 halves down its column. Consecutive threads
// take consecutive columns, so each row of stores of a wave is contiguous.
// This is a one-off HBM stream (2 bytes written per weight). With bf16 data
// (scales, zero points and the output in bfloat16) the fp64 product is rounded
// once to bf16: first to binary32 rounding to odd (truncate, then set the last
// bit if anything was dropped), then to bf16 to nearest even, which equals one
// direct rounding since binary32 keeps more than two extra bits.
#include "common.h"

namespace qmm {
namespace {

constexpr int kThreads = 256;

// Words of the main plane per 32 codes.
template <int BITS> constexpr int words_per_chunk() { return BITS == 3 ? 2 : BITS; }

template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&wd)[words_per_chunk<BITS>()], uint32_t lo, int k) {
  if constexpr (BITS == 3) {
    return (((wd[k >> 4] >> (2 * (k & 15))) & 3u) << 1) | ((lo >> k) & 1u);
  } else {
    constexpr int EPS = 32 / BITS;
    return (wd[k / EPS] >> ((k % EPS) * BITS)) & ((1u << BITS) - 1u);
  }
}

// fp64 -> bf16 bits, rounded once to nearest even (finite values). Below
// 2^-126 bf16 has fixed spacing 2^-133 and the bit pattern is the number of
// those units, rounded to nearest even, here in fp64 so that the result does
// not depend on how binary32 denormals are treated.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double d) {
  const double mag = __builtin_fabs(d);
  if (mag < 0x1p-126) {
    const uint32_t units = (uint32_t)__builtin_rint(mag * 0x1p133);  // 0 .. 128, exact scaling
    return (uint16_t)(units | (__builtin_signbit(d) ? 0x8000u : 0u));
  }
  const float f = (float)d;  // nearest binary32
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  const double back = (double)f;
  if (back != d) {
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;  // truncate: one step toward zero
    u |= 1u;                                                 // round to odd
  }
  u += 0x7FFFu + ((u >> 16) & 1u);  // nearest even at 16 bits
  return (uint16_t)(u >> 16);
}

template <int BITS, bool BF>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint32_t* __restrict__ qw,
                                                           const uint32_t* __restrict__ qlo,
                                                           const uint16_t* __restrict__ zeros,
                                                           const uint16_t* __restrict__ scales, int K, int N,
                                                           int rows_per_group, uint16_t* __restrict__ w) {
  constexpr int NWORDS = words_per_chunk<BITS>();
  const long long total = (long long)(K / 32) * N;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i / N);  // 32-row chunk
  const int n = (int)(i - (long long)c * N);
  uint32_t wd[NWORDS];
#pragma unroll
  for (int r = 0; r < NWORDS; ++r) wd[r] = qw[(size_t)(c * NWORDS + r) * N + n];
  const uint32_t lo = BITS == 3 ? qlo[(size_t)c * N + n] : 0u;
  const int g = (32 * c) / rows_per_group;
  const double s = (double)bits_to_float<BF>(scales[(size_t)g * N + n]);
  const double z = (double)bits_to_float<BF>(zeros[(size_t)g * N + n]);
  uint16_t* col = w + (size_t)32 * c * N + n;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const double v = ((double)code_at<BITS>(wd, lo, k) - z) * s;
    col[(size_t)k * N] = BF ? f64_to_bf16_bits(v) : __builtin_bit_cast(uint16_t, (f16)v);
  }
}

template <int BITS, bool BF>
hipError_t launch_typed(const uint32_t* qw, const uint32_t* qlo, const uint16_t* zeros, const uint16_t* scales,
                        int K, int N, int rows_per_group, uint16_t* w, hipStream_t s) {
  const long long total = (long long)(K / 32) * N;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
  dequant_kernel<BITS, BF><<<blocks, kThreads, 0, s>>>(qw, qlo, zeros, scales, K, N, rows_per_group, w);
  return hipGetLastError();
}

template <bool BF>
hipError_t launch_dtype(const uint32_t* qw, const uint32_t* qlo, const uint16_t* zeros, const uint16_t* scales,
                        int K, int N, int bits, int rows, uint16_t* w, hipStream_t s) {
  switch (bits) {
    case 1: return launch_typed<1, BF>(qw, qlo, zeros, scales, K, N, rows, w, s);
    case 2: return launch_typed<2, BF>(qw, qlo, zeros, scales, K, N, rows, w, s);
    case 3: return launch_typed<3, BF>(qw, qlo, zeros, scales, K, N, rows, w, s);
    case 4: return launch_typed<4, BF>(qw, qlo, zeros, scales, K, N, rows, w, s);
    case 8: return launch_typed<8, BF>(qw, qlo, zeros, scales, K, N, rows, w, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_dequant(const uint32_t* qw, const uint32_t* qlo, const uint16_t* zeros,
                          const uint16_t* scales, int K, int N, int bits, int group_size, uint16_t* w,
                          bool bf16, hipStream_t s) {
  const int rows = group_rows(K, group_size);
  return bf16 ? launch_dtype<true>(qw, qlo, zeros, scales, K, N, bits, rows, w, s)
              : launch_dtype<false>(qw, qlo, zeros, scales, K, N, bits, rows, w, s);
}

}  // namespace qmm
