// K-major packing of integer codes into 32-bit words and its inverse.
//
// Layout (dashq_kernel.py, module docstring and _pack_kmajor / _unpack_kmajor):
// codes (K, N) row-major; words (K / eps, N), eps = 32 / bits; code k of
// column n sits in word k / eps of column n at bit offset (k % eps) * bits.
// 3-bit codes are two planes (TritonQuantLinear.__init__): a 2-bit plane of
// q >> 1 and a 1-bit plane of q & 1. Widths 1, 2, 3, 4 and 8 (SUPPORTED_NBITS).
//
// One thread per output word (pack) or per input word (unpack); consecutive
// threads take consecutive columns, so every global access is coalesced along
// N. These run once when weights are loaded; they are plain HBM streams.
#include "common.h"

namespace qmm {
namespace {

constexpr int kThreads = 256;

// Pack one plane: word (r, n) gathers codes k = r * EPS + j, j < EPS, after
// applying `shift` and masking to BITS bits. `shift` selects the part of a
// 3-bit code a plane holds (1 for the high plane, 0 otherwise).
template <int BITS>
__global__ __launch_bounds__(kThreads) void pack_plane_kernel(const uint8_t* __restrict__ codes, int K,
                                                              int N, int shift, int code_bits,
                                                              uint32_t* __restrict__ words,
                                                              int32_t* __restrict__ bad_count) {
  constexpr int EPS = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const long long total = (long long)(K / EPS) * N;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int r = (int)(i / N);
  const int n = (int)(i - (long long)r * N);
  const uint8_t* col = codes + (size_t)r * EPS * N + n;
  uint32_t w = 0;
  int bad = 0;
#pragma unroll
  for (int j = 0; j < EPS; ++j) {
    const uint32_t q = col[(size_t)j * N];
    bad += (q >> code_bits) != 0;
    w |= ((q >> shift) & MASK) << (j * BITS);
  }
  words[i] = w;
  if (bad_count != nullptr && bad != 0) atomicAdd(bad_count, bad);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void unpack_plane_kernel(const uint32_t* __restrict__ words, int K,
                                                                int N, uint8_t* __restrict__ codes) {
  constexpr int EPS = 32 / BITS;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const long long total = (long long)(K / EPS) * N;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int r = (int)(i / N);
  const int n = (int)(i - (long long)r * N);
  const uint32_t w = words[i];
  uint8_t* col = codes + (size_t)r * EPS * N + n;
#pragma unroll
  for (int j = 0; j < EPS; ++j) col[(size_t)j * N] = (uint8_t)((w >> (j * BITS)) & MASK);
}

// 3-bit: q = (hi << 1) | lo, hi from the 2-bit plane (16 per word), lo from the
// 1-bit plane (32 per word). One thread per 1-bit word, i.e. 32 codes.
__global__ __launch_bounds__(kThreads) void unpack3_kernel(const uint32_t* __restrict__ hi_words,
                                                           const uint32_t* __restrict__ lo_words, int K,
                                                           int N, uint8_t* __restrict__ codes) {
  const long long total = (long long)(K / 32) * N;
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int r = (int)(i / N);
  const int n = (int)(i - (long long)r * N);
  const uint32_t lo = lo_words[i];
  const uint32_t h0 = hi_words[(size_t)(2 * r) * N + n];
  const uint32_t h1 = hi_words[(size_t)(2 * r + 1) * N + n];
  uint8_t* col = codes + (size_t)r * 32 * N + n;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t h = ((j < 16 ? h0 : h1) >> (2 * (j & 15))) & 3u;
    col[(size_t)j * N] = (uint8_t)((h << 1) | ((lo >> j) & 1u));
  }
}

inline unsigned blocks_for(long long n) { return (unsigned)((n + kThreads - 1) / kThreads); }

template <int BITS>
hipError_t pack_plane(const uint8_t* codes, int K, int N, int shift, int code_bits, uint32_t* words,
                      int32_t* bad, hipStream_t s) {
  const long long total = (long long)(K / (32 / BITS)) * N;
  if (total == 0) return hipSuccess;
  pack_plane_kernel<BITS><<<blocks_for(total), kThreads, 0, s>>>(codes, K, N, shift, code_bits, words, bad);
  return hipGetLastError();
}

template <int BITS>
hipError_t unpack_plane(const uint32_t* words, int K, int N, uint8_t* codes, hipStream_t s) {
  const long long total = (long long)(K / (32 / BITS)) * N;
  if (total == 0) return hipSuccess;
  unpack_plane_kernel<BITS><<<blocks_for(total), kThreads, 0, s>>>(words, K, N, codes);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, int K, int N, int bits, uint32_t* qw, uint32_t* qlo,
                       int32_t* bad_count, hipStream_t s) {
  switch (bits) {
    case 1: return pack_plane<1>(codes, K, N, 0, 1, qw, bad_count, s);
    case 2: return pack_plane<2>(codes, K, N, 0, 2, qw, bad_count, s);
    case 4: return pack_plane<4>(codes, K, N, 0, 4, qw, bad_count, s);
    case 8: return pack_plane<8>(codes, K, N, 0, 8, qw, bad_count, s);
    case 3: {
      // Out-of-range codes are counted once, by the high plane's pass.
      hipError_t e = pack_plane<2>(codes, K, N, 1, 3, qw, bad_count, s);
      if (e != hipSuccess) return e;
      return pack_plane<1>(codes, K, N, 0, 8, qlo, nullptr, s);
    }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_unpack(const uint32_t* qw, const uint32_t* qlo, int K, int N, int bits, uint8_t* codes,
                         hipStream_t s) {
  switch (bits) {
    case 1: return unpack_plane<1>(qw, K, N, codes, s);
    case 2: return unpack_plane<2>(qw, K, N, codes, s);
    case 4: return unpack_plane<4>(qw, K, N, codes, s);
    case 8: return unpack_plane<8>(qw, K, N, codes, s);
    case 3: {
      const long long total = (long long)(K / 32) * N;
      if (total == 0) return hipSuccess;
      unpack3_kernel<<<blocks_for(total), kThreads, 0, s>>>(qw, qlo, K, N, codes);
      return hipGetLastError();
    }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
