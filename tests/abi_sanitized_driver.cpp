// Host-side exercise of the C ABI for the address and undefined-behaviour
// sanitizers: every call below is refused by argument validation (no kernel
// is launched), plus the host-only queries (status strings, workspace sizes,
// launch plans) over ordinary and extreme arguments. Built and run by
// tests/test_abi_sanitized.py against a library whose host code carries the
// sanitizers. Exit status 0 when every status matches.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qmm.h"

static int failures = 0;

#define EXPECT(call, want)                                                                       \
  do {                                                                                           \
    const int got_ = (int)(call);                                                                \
    if (got_ != (int)(want)) {                                                                   \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, got_, \
              (int)(want), qmm_last_error());                                                    \
      ++failures;                                                                                \
    }                                                                                            \
    const size_t len_ = strlen(qmm_last_error());                                                \
    if ((int)(want) != QMM_OK && (len_ == 0 || len_ >= 512)) {                                   \
      fprintf(stderr, "%s:%d: error message of length %zu\n", __FILE__, __LINE__, len_);         \
      ++failures;                                                                                \
    }                                                                                            \
  } while (0)

// Fake device addresses, never dereferenced: every call fails validation first.
static void* const A = (void*)0x10000;
static void* const MIS = (void*)0x10004;
#define P(T) ((T*)A)
#define PM(T) ((T*)MIS)

static void products(void) {
  typedef qmm_status (*gemv_fn)(const uint16_t*, int, int, const int32_t*, const int32_t*, const uint16_t*,
                                const uint16_t*, const uint16_t*, int, int, int, uint16_t*, void*, size_t,
                                hipStream_t);
  typedef qmm_status (*gemm_fn)(const uint16_t*, int, int, const int32_t*, const int32_t*, const uint16_t*,
                                const uint16_t*, const uint16_t*, int, int, int, uint16_t*, hipStream_t);
  const gemv_fn gemvs[2] = {qmm_gemv, qmm_gemv_bf16};
  const gemm_fn gemms[2] = {qmm_gemm, qmm_gemm_bf16};
  const uint16_t* x = P(const uint16_t);
  const int32_t* qw = P(const int32_t);
  const uint16_t* z = P(const uint16_t);
  uint16_t* y = P(uint16_t);
  for (int f = 0; f < 2; ++f) {
    gemv_fn g = gemvs[f];
    EXPECT(g(x, 1, 256, qw, qw, z, z, nullptr, 64, 5, 128, y, A, 1 << 30, nullptr), QMM_ERR_BITS);
    EXPECT(g(x, 0, 256, qw, qw, z, z, nullptr, 64, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, 17, 256, qw, qw, z, z, nullptr, 64, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, INT_MIN, 256, qw, qw, z, z, nullptr, 64, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, 1, 48, qw, qw, z, z, nullptr, 64, 4, -1, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, 1, INT_MAX, qw, qw, z, z, nullptr, 64, 4, -1, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, 1, 256, qw, qw, z, z, nullptr, 60, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, 1, 256, qw, qw, z, z, nullptr, INT_MAX, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, 1, 256, qw, qw, z, z, nullptr, (1 << 20) + 8, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(g(x, 1, 256, qw, qw, z, z, nullptr, 64, 4, 48, y, A, 1 << 30, nullptr), QMM_ERR_GROUP);
    EXPECT(g(x, 1, 256, qw, qw, z, z, nullptr, 64, 4, INT_MIN, y, A, 1 << 30, nullptr), QMM_ERR_GROUP);
    EXPECT(g(nullptr, 1, 256, qw, qw, z, z, nullptr, 64, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_NULL);
    EXPECT(g(x, 1, 256, qw, nullptr, z, z, nullptr, 64, 3, 128, y, A, 1 << 30, nullptr), QMM_ERR_NULL);
    EXPECT(g(x, 1, 256, qw, qw, z, z, nullptr, 64, 4, 128, nullptr, A, 1 << 30, nullptr), QMM_ERR_NULL);
    EXPECT(g(PM(const uint16_t), 1, 256, qw, qw, z, z, nullptr, 64, 4, 128, y, A, 1 << 30, nullptr), QMM_ERR_ALIGN);
    EXPECT(g(x, 1, 256, qw, qw, z, z, (const uint16_t*)((char*)A + 1), 64, 4, 128, y, A, 1 << 30, nullptr),
           QMM_ERR_ALIGN);
    EXPECT(g(x, 16, 65536, qw, qw, z, z, nullptr, 64, 4, -1, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    // a deep, narrow product needs a workspace
    EXPECT(g(x, 1, 8192, qw, qw, z, z, nullptr, 64, 4, 128, y, nullptr, 0, nullptr), QMM_ERR_WORKSPACE);
    EXPECT(g(x, 1, 8192, qw, qw, z, z, nullptr, 64, 4, 128, y, A, 16, nullptr), QMM_ERR_WORKSPACE);
    EXPECT(g(x, 1, 8192, qw, qw, z, z, nullptr, 64, 4, 128, y, MIS, 1 << 30, nullptr), QMM_ERR_ALIGN);

    gemm_fn h = gemms[f];
    EXPECT(h(x, 300, 256, qw, qw, z, z, nullptr, 64, 6, 128, y, nullptr), QMM_ERR_BITS);
    EXPECT(h(x, -1, 256, qw, qw, z, z, nullptr, 64, 4, 128, y, nullptr), QMM_ERR_SHAPE);
    EXPECT(h(x, INT_MAX, INT_MAX - 31, qw, qw, z, z, nullptr, 64, 4, -1, y, nullptr), QMM_ERR_SHAPE);
    EXPECT(h(x, 1 << 17, 16384, qw, qw, z, z, nullptr, 64, 4, -1, y, nullptr), QMM_ERR_SHAPE);
    EXPECT(h(x, 300, 256, qw, qw, z, z, nullptr, 64, 4, 0, y, nullptr), QMM_ERR_GROUP);
    EXPECT(h(x, 300, 256, qw, qw, nullptr, z, nullptr, 64, 4, 128, y, nullptr), QMM_ERR_NULL);
    EXPECT(h(x, 300, 256, qw, qw, PM(const uint16_t), z, nullptr, 64, 4, 128, y, nullptr), QMM_ERR_ALIGN);
  }
  EXPECT(qmm_gemv_noalloc(x, 1, 256, qw, qw, z, z, nullptr, 64, 5, 128, y, nullptr), QMM_ERR_BITS);
  EXPECT(qmm_gemv_noalloc(x, 1, 256, qw, qw, z, z, nullptr, 64, 4, 128, nullptr, nullptr), QMM_ERR_NULL);

  // The flags entry points: unknown bits first, then the checks of the plain calls.
  for (unsigned fl : {4u, 8u, 0x80000000u, 0xffffffffu}) {
    EXPECT(qmm_gemv_ex(x, 1, 256, qw, qw, z, z, nullptr, 64, 4, 128, fl, y, A, 1 << 30, nullptr), QMM_ERR_FLAGS);
    EXPECT(qmm_gemm_ex(x, 300, 256, qw, qw, z, z, nullptr, 64, 4, 128, fl, y, nullptr), QMM_ERR_FLAGS);
  }
  for (unsigned fl : {0u, QMM_BF16, QMM_STRIPS, QMM_BF16 | QMM_STRIPS}) {
    EXPECT(qmm_gemv_ex(x, 1, 256, qw, qw, z, z, nullptr, 64, 5, 128, fl, y, A, 1 << 30, nullptr), QMM_ERR_BITS);
    EXPECT(qmm_gemv_ex(x, 17, 256, qw, qw, z, z, nullptr, 64, 4, 128, fl, y, A, 1 << 30, nullptr), QMM_ERR_SHAPE);
    EXPECT(qmm_gemv_ex(x, 1, 256, qw, qw, z, z, nullptr, 64, 4, 128, fl, nullptr, A, 1 << 30, nullptr), QMM_ERR_NULL);
    EXPECT(qmm_gemv_ex(x, 1, 8192, qw, qw, z, z, nullptr, 64, 4, 128, fl, y, nullptr, 0, nullptr), QMM_ERR_WORKSPACE);
    EXPECT(qmm_gemm_ex(x, 300, 256, qw, qw, z, z, nullptr, 64, 4, 0, fl, y, nullptr), QMM_ERR_GROUP);
    EXPECT(qmm_gemm_ex(x, 300, 256, qw, qw, PM(const uint16_t), z, nullptr, 64, 4, 128, fl, y, nullptr), QMM_ERR_ALIGN);
  }
  // A plane that fits K-major (K * N bytes < 4 GiB) but not once N = 8 is
  // padded to a 16-column strip.
  EXPECT(qmm_gemm_ex(x, 1, 1 << 28, qw, qw, z, z, nullptr, 8, 8, -1, QMM_STRIPS, y, nullptr), QMM_ERR_SHAPE);
  EXPECT(qmm_gemv_ex(x, 1, 1 << 28, qw, qw, z, z, nullptr, 8, 8, -1, QMM_STRIPS, y, A, 1 << 30, nullptr),
         QMM_ERR_SHAPE);
}

static void conversions(void) {
  const uint8_t* codes = P(const uint8_t);
  int32_t* qw = P(int32_t);
  EXPECT(qmm_pack(codes, 64, 8, 5, qw, qw, nullptr, nullptr), QMM_ERR_BITS);
  EXPECT(qmm_pack(codes, 12, 8, 4, qw, nullptr, nullptr, nullptr), QMM_ERR_SHAPE);
  EXPECT(qmm_pack(codes, INT_MAX, INT_MAX, 4, qw, nullptr, nullptr, nullptr), QMM_ERR_SHAPE);
  EXPECT(qmm_pack(codes, 64, 8, 3, qw, nullptr, nullptr, nullptr), QMM_ERR_NULL);
  EXPECT(qmm_pack(nullptr, 64, 8, 4, qw, nullptr, nullptr, nullptr), QMM_ERR_NULL);
  EXPECT(qmm_unpack(qw, nullptr, 64, 8, 4, nullptr, nullptr), QMM_ERR_NULL);
  EXPECT(qmm_unpack(qw, nullptr, -32, 8, 4, P(uint8_t), nullptr), QMM_ERR_SHAPE);
  const uint16_t* z = P(const uint16_t);
  EXPECT(qmm_dequant(qw, qw, z, z, 256, 64, 5, 128, P(uint16_t), nullptr), QMM_ERR_BITS);
  EXPECT(qmm_dequant(qw, qw, z, z, 256, 64, 4, 48, P(uint16_t), nullptr), QMM_ERR_GROUP);
  EXPECT(qmm_dequant_bf16(qw, qw, z, z, 256, 64, 4, 128, (uint16_t*)((char*)A + 1), nullptr), QMM_ERR_ALIGN);
  int32_t* st = P(int32_t);
  for (int dir = 0; dir < 2; ++dir) {
    auto f = dir == 0 ? qmm_to_strips : qmm_from_strips;
    EXPECT(f(qw, 0, 64, st, nullptr), QMM_ERR_SHAPE);
    EXPECT(f(qw, 16, INT_MIN, st, nullptr), QMM_ERR_SHAPE);
    EXPECT(f(qw, INT_MAX, INT_MAX, st, nullptr), QMM_ERR_SHAPE);
    EXPECT(f(qw, 1 << 26, 24, st, nullptr), QMM_ERR_SHAPE);  // 2^26 * 32 * 4 bytes = 8 GiB
    EXPECT(f(nullptr, 16, 64, st, nullptr), QMM_ERR_NULL);
    EXPECT(f(qw, 16, 64, nullptr, nullptr), QMM_ERR_NULL);
    EXPECT(f(qw, 16, 64, (int32_t*)((char*)A + 2), nullptr), QMM_ERR_ALIGN);
  }
}

static void queries(void) {
  if (qmm_abi_version() != QMM_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", qmm_abi_version(), QMM_ABI_VERSION);
    ++failures;
  }
  for (int s = -2; s < 12; ++s) {
    const char* name = qmm_status_string(s);
    if (name == nullptr || strncmp(name, "QMM_", 4) != 0) {
      fprintf(stderr, "status string of %d\n", s);
      ++failures;
    }
  }
  // Workspace sizes and plans over ordinary and extreme shapes: only the
  // arithmetic runs (the sanitizers watch it).
  const int Ms[] = {INT_MIN, -1, 0, 1, 2, 8, 16, 17, 2048, INT_MAX};
  const int Ks[] = {INT_MIN, 0, 32, 96, 4096, 14336, 65536, 1 << 24, INT_MAX - 31, INT_MAX};
  const int Ns[] = {INT_MIN, 0, 8, 136, 4096, 11008, 1 << 20, (1 << 20) + 8, 1 << 30, INT_MAX - 7};
  const int bits[] = {0, 1, 2, 3, 4, 5, 8, 16};
  const int gss[] = {INT_MIN, -1, 0, 32, 128, 4096, INT_MAX};
  int32_t info[16];
  size_t total = 0;
  for (int M : Ms)
    for (int K : Ks)
      for (int N : Ns)
        for (int b : bits)
          for (int gs : gss) {
            total += qmm_workspace_bytes(M, K, N, b, gs);
            const qmm_status st = qmm_gemv_plan_info(M, K, N, b, gs, info, 16);
            if (st == QMM_OK && (info[1] < 1 || info[2] < 1 || info[3] < 1 || info[4] < 1)) {
              fprintf(stderr, "gemv plan %d %d %d %d %d: %d %d %d %d\n", M, K, N, b, gs, info[1], info[2], info[3],
                      info[4]);
              ++failures;
            }
            const qmm_status st2 = qmm_gemm_plan_info(M, K, N, b, gs, info, 16);
            if (st2 == QMM_OK && (info[0] < 64 || info[1] < 64 || info[4] < 1)) {
              fprintf(stderr, "gemm plan %d %d %d %d %d\n", M, K, N, b, gs);
              ++failures;
            }
          }
  EXPECT(qmm_gemv_plan_info(1, 4096, 4096, 4, 128, nullptr, 9), QMM_ERR_NULL);
  EXPECT(qmm_gemm_plan_info(2048, 4096, 14336, 8, -1, nullptr, 7), QMM_ERR_NULL);
  EXPECT(qmm_gemv_plan_info(1, 4096, 4096, 4, 128, info, 9), QMM_OK);
  EXPECT(qmm_gemm_plan_info(2048, 4096, 14336, 8, -1, info, 7), QMM_OK);
  const int rws[] = {INT_MIN, -1, 0, 1, 2, 255, 1 << 20, 1 << 26, INT_MAX};
  const int cols[] = {INT_MIN, -1, 0, 1, 8, 15, 16, 17, 4104, 1 << 20, INT_MAX - 14, INT_MAX};
  for (int r : rws)
    for (int c : cols) {
      const size_t b = qmm_strips_bytes(r, c);
      const bool fits = r >= 1 && c >= 1 && (unsigned long long)r * ((c + 15ull) / 16 * 16) * 4 < (1ull << 32);
      if (fits != (b > 0) || (fits && b != (size_t)r * ((c + 15ull) / 16 * 16) * 4)) {
        fprintf(stderr, "strips bytes %d %d: %zu\n", r, c, b);
        ++failures;
      }
    }
  printf("workspace bytes summed over the sweep: %zu\n", total);
}

int main() {
  products();
  conversions();
  queries();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("all calls refused or answered as expected\n");
  return 0;
}
