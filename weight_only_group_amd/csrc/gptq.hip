// GPTQModel-format inputs converted into this library's layouts, once, when
// weights are loaded.
//
// GPTQModel-Compatible Triton Kernel README, "API Reference" (qzeros: the
// packed quantized zero points) and "Quantization Format" (int32 words of 16,
// 10, 8 or 4 values for 2, 3, 4 or 8 bits, the 3-bit words padded). The README
// does not place the values. Read here as: value i of a word at bit offset
// i * bits, lowest first (a 3-bit word holds 10 values in bits 0-29 and leaves
// bits 30-31 unused); weights packed along K, zero points along N, the last
// word of a row or column partly filled. In that reading 2-, 4- and 8-bit
// weight words are already the K-major words the products read, so only the
// zero points and the 3-bit weights need converting.
//
// Both kernels are plain HBM streams: one thread per output element (zero
// points) or per 32-row block of a column (3-bit planes), consecutive threads
// on consecutive columns, so every global access is coalesced along N.
#include "gptq.h"

namespace qmm {
namespace {

constexpr int kThreads = 256;

template <bool BF>
__global__ __launch_bounds__(kThreads) void unpack_qzeros_kernel(const uint32_t* __restrict__ qz, int G, int N,
                                                                 int words_per_row, int bits, int per_word,
                                                                 uint16_t* __restrict__ zeros) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (long long)G * N) return;
  const int g = (int)(i / N);
  const int n = (int)(i - (long long)g * N);
  const uint32_t w = qz[(size_t)g * words_per_row + n / per_word];
  const uint32_t z = (w >> ((n % per_word) * bits)) & ((1u << bits) - 1u);
  zeros[i] = float_to_bits<BF>((float)z);  // an integer below 256: exact in fp16 and bf16
}

// Codes k = 32 r .. 32 r + 31 of column n lie in at most four 10-value words,
// starting at word 32 r / 10 with slot 32 r % 10. They are written as the two
// planes qmm_pack writes: the 2-bit plane of q >> 1 (16 per word, rows 2 r and
// 2 r + 1) and the 1-bit plane of q & 1 (32 per word, row r).
__global__ __launch_bounds__(kThreads) void repack_3bit10_kernel(const uint32_t* __restrict__ w10, int K, int N,
                                                                 uint32_t* __restrict__ plane2,
                                                                 uint32_t* __restrict__ plane1) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (long long)(K / 32) * N) return;
  const int r = (int)(i / N);
  const int n = (int)(i - (long long)r * N);
  const int rows10 = (K + 9) / 10;
  const int first = (32 * r) / 10;
  uint32_t wv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = first + t;
    wv[t] = row < rows10 ? w10[(size_t)row * N + n] : 0u;
  }
  uint32_t h0 = 0, h1 = 0, lo = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const int k = 32 * r + j;
    const int t = k / 10 - first;  // 0..3
    const uint32_t w = t == 0 ? wv[0] : (t == 1 ? wv[1] : (t == 2 ? wv[2] : wv[3]));
    const uint32_t q = (w >> (3 * (k % 10))) & 7u;
    if (j < 16) h0 |= (q >> 1) << (2 * j);
    else h1 |= (q >> 1) << (2 * (j - 16));
    lo |= (q & 1u) << j;
  }
  plane2[(size_t)(2 * r) * N + n] = h0;
  plane2[(size_t)(2 * r + 1) * N + n] = h1;
  plane1[(size_t)r * N + n] = lo;
}

unsigned blocks_for(long long n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

int gptq_values_per_word(int bits) { return bits == 3 ? 10 : 32 / bits; }

hipError_t launch_unpack_qzeros(const uint32_t* qzeros, int G, int N, int bits, uint16_t* zeros, bool bf16,
                                hipStream_t s) {
  const int e = gptq_values_per_word(bits);
  const int words_per_row = (N + e - 1) / e;
  const long long total = (long long)G * N;
  if (bf16)
    unpack_qzeros_kernel<true><<<blocks_for(total), kThreads, 0, s>>>(qzeros, G, N, words_per_row, bits, e, zeros);
  else
    unpack_qzeros_kernel<false><<<blocks_for(total), kThreads, 0, s>>>(qzeros, G, N, words_per_row, bits, e, zeros);
  return hipGetLastError();
}

hipError_t launch_repack_3bit10(const uint32_t* w10, int K, int N, uint32_t* plane2, uint32_t* plane1,
                                hipStream_t s) {
  const long long total = (long long)(K / 32) * N;
  repack_3bit10_kernel<<<blocks_for(total), kThreads, 0, s>>>(w10, K, N, plane2, plane1);
  return hipGetLastError();
}

}  // namespace qmm
