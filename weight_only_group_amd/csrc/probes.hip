// Reference kernels for measurement only (libqmm_probes.so, not part of the
// qmm ABI): the floors the quantized-matmul kernels are judged against.
//
//  qmm_probe_empty  - a kernel that does nothing: the dispatch floor of a
//                     launch of a given shape (as a graph node, back to back).
//  qmm_probe_read   - a plain streaming read of `bytes` bytes with 16-byte
//                     non-temporal loads (the same load width and cache hint
//                     the GEMV uses).
//  qmm_probe_mfma   - a dense loop of independent V_MFMA_F32_32X32X16_F16 per
//                     wave, registers only: the matrix-core peak reachable
//                     from a kernel.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void empty_kernel() {}

__global__ void read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // A store that depends on every thread's words keeps every load; it happens
  // only for one particular value (harmless when it does).
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink) {
  f16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(threadIdx.x * 0.001f + e);
    b[e] = (_Float16)(e * 0.5f);
  }
  f32x16 acc[4];
  for (int t = 0; t < 4; ++t)
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[t], 0, 0, 0);
  }
  float s = 0.f;
  for (int t = 0; t < 4; ++t)
    for (int r = 0; r < 16; ++r) s += acc[t][r];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // never true for these inputs; keeps the loop
}

}  // namespace

extern "C" {

int qmm_probe_empty(int blocks, int threads, hipStream_t stream) {
  if (blocks < 1 || threads < 1 || threads > 1024) return 1;
  empty_kernel<<<blocks, threads, 0, stream>>>();
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

// p: device buffer of `bytes` bytes (multiple of 16, 16-byte aligned); sink:
// device array of at least `blocks` words.
int qmm_probe_read(const void* p, size_t bytes, int blocks, int threads, uint32_t* sink, hipStream_t stream) {
  if (!p || !sink || bytes % 16 != 0 || ((uintptr_t)p & 15) != 0 || blocks < 1 || threads < 64 || threads > 1024)
    return 1;
  read_kernel<<<blocks, threads, 0, stream>>>(static_cast<const u32x4*>(p), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

// 4 waves per block; each wave issues 4 * iters MFMAs of 2 * 32 * 32 * 16 flops.
int qmm_probe_mfma(int blocks, int iters, float* sink, hipStream_t stream) {
  if (!sink || blocks < 1 || iters < 1) return 1;
  mfma_kernel<<<blocks, 256, 0, stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
