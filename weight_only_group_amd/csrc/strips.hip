// Load-time re-layout of packed word planes into 16-column strips, and back.
//
// The products read a plane of packed words (rows x N int32, the K-major
// packing of their inputs) column strip by column strip: the decode product
// gives each block one strip of 16 columns over all of K. In the K-major
// layout such a strip is a 64-byte piece of every row, rows N * 4 bytes
// apart; in the strip-major layout each strip is one contiguous run (word
// (r, n) at ((n / 16) * rows + r) * 16 + n % 16), so a block streams its
// words in order. The words themselves, and so every result of the products,
// are unchanged: this is a permutation, with the last strip's columns past N
// padded with zeros. It runs once when weights are loaded (a plain HBM
// stream): one thread per output word, consecutive threads on consecutive
// output words.
#include "common.h"

namespace qmm {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void to_strips_kernel(const uint32_t* __restrict__ words, int rows, int N,
                                                              uint32_t* __restrict__ strips, size_t total) {
  const size_t o = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (o >= total) return;
  const size_t per_strip = (size_t)rows * kStripCols;
  const int s = (int)(o / per_strip);
  const int rem = (int)(o - (size_t)s * per_strip);
  const int r = rem / kStripCols, c = rem % kStripCols;
  const int n = s * kStripCols + c;
  strips[o] = n < N ? words[(size_t)r * N + n] : 0u;
}

__global__ __launch_bounds__(kThreads) void from_strips_kernel(const uint32_t* __restrict__ strips, int rows, int N,
                                                                uint32_t* __restrict__ words, size_t total) {
  const size_t o = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (o >= total) return;
  const int r = (int)(o / (size_t)N), n = (int)(o - (size_t)r * N);
  words[o] = strips[((size_t)(n / kStripCols) * rows + r) * kStripCols + n % kStripCols];
}

unsigned blocks_for(size_t total) { return (unsigned)((total + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_to_strips(const uint32_t* words, int rows, int N, uint32_t* strips, hipStream_t s) {
  const size_t total = (size_t)rows * plane_cols(N, 1);
  to_strips_kernel<<<blocks_for(total), kThreads, 0, s>>>(words, rows, N, strips, total);
  return hipGetLastError();
}

hipError_t launch_from_strips(const uint32_t* strips, int rows, int N, uint32_t* words, hipStream_t s) {
  const size_t total = (size_t)rows * N;
  from_strips_kernel<<<blocks_for(total), kThreads, 0, s>>>(strips, rows, N, words, total);
  return hipGetLastError();
}

}  // namespace qmm
