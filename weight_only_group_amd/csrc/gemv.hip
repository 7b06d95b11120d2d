// Decode product y = x @ dequant(W) for 1 <= M <= 16 on gfx950.
//
// What is computed (GPTQModel-Compatible Triton Kernel README, "API
// Reference" and "Dequantization Formula"; dashq_kernel.py, _dashq_gemv_kernel):
//   y[m, n] = sum_g scale[g, n] * sum_{k in g} x[m, k] * (q[k, n] - zero[g, n])
// over K-major packed words. The page's GEMV reads every packed word once with
// coalesced loads, fetches one scale/zero pair per group and combines split-K
// pieces with float atomics. This kernel keeps the first two ideas and
// replaces the rest:
//
//  * A wave owns 16 * VEC adjacent columns. Lane l loads VEC adjacent words of
//    one word row (one 8- or 16-byte load; a wave row segment is 128 or 256
//    contiguous bytes) with a non-temporal hint, since weights are streamed
//    once.
//  * Codes become halves with one AND-OR into the mantissa of 1024.0 (exact),
//    then one packed subtract of (1024 + zero) when the zero point is an
//    integer (exact), else two subtracts.
//  * The multiply-accumulate runs on the matrix cores: V_MFMA_F32_16X16X32_F16
//    with x as the 16 x 32 A operand (rows >= M are zero) and the dequantized
//    codes as the 32 x 16 B operand. Lane group j = l / 16 of the wave feeds
//    8 of the 32 k values of a "unit" (32 consecutive k), so a unit never
//    straddles a group (group_size % 32 == 0) and the fp32 accumulator of a
//    group is multiplied by that group's scale once (exact dequantized values
//    up to the scale product).
//  * Waves of a block take consecutive K ranges of the same column strip and
//    are summed through LDS in wave order. Blocks along K write fp32 partial
//    sums; the last block of a strip to arrive (an atomic ticket) adds the
//    partials in split order and writes fp16 (round to nearest even). The sum
//    order never depends on arrival order, so results are bitwise repeatable,
//    and the ticket is reset to zero by that block.
#include <type_traits>

#include "common.h"

#ifndef QMM_GEMV_TARGET_WAVES
#define QMM_GEMV_TARGET_WAVES 2048  // waves in flight to aim for (8 per CU)
#endif
#ifndef QMM_GEMV_VEC
#define QMM_GEMV_VEC 0  // 0: chosen per shape
#endif
#ifndef QMM_GEMV_WAVES
#define QMM_GEMV_WAVES 0  // 0: chosen per shape
#endif
#ifndef QMM_GEMV_XCD_REMAP
#define QMM_GEMV_XCD_REMAP 1
#endif

namespace qmm {
namespace {

constexpr int kMaxM = 16;
constexpr int kMaxSplit = 16;  // blocks along K per column strip
constexpr int kCUs = 256;      // compute units of an MI355X
// Arrival counters live in a fixed header at the start of the workspace, one
// per column strip, and partial sums start after it. The header never
// overlaps any call's partial sums, so counters left at zero by one call are
// still zero for the next call, whatever the two shapes are.
constexpr size_t kCounterHeaderBytes = size_t(kGemvMaxStrips) * 4;

// Words per lane per unit and column: 4-bit 1 row, 8-bit 2 rows, 2-bit 1 row
// (two lane groups share it), 3-bit one word of each plane.
template <int BITS> struct Bits;
template <> struct Bits<4> { static constexpr int NW = 1; };
template <> struct Bits<8> { static constexpr int NW = 2; };
template <> struct Bits<2> { static constexpr int NW = 1; };
template <> struct Bits<3> { static constexpr int NW = 2; };

template <int VEC> struct Vec;
template <> struct Vec<1> { typedef uint32_t T; };
template <> struct Vec<2> { typedef u32x2 T; };
template <> struct Vec<4> { typedef u32x4 T; };

template <int VEC>
__device__ __forceinline__ uint32_t word_at(typename Vec<VEC>::T w, int v) {
  if constexpr (VEC == 1) return w;
  else return w[v];
}

template <int VEC>
__device__ __forceinline__ typename Vec<VEC>::T load_words(const uint32_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename Vec<VEC>::T*>(p));
}

// Row (in its plane) of word w of unit u for lane group j.
template <int BITS>
__device__ __forceinline__ int word_row(int u, int j, int w) {
  if constexpr (BITS == 4) return 4 * u + j;
  else if constexpr (BITS == 8) return 8 * u + 2 * j + w;
  else if constexpr (BITS == 2) return 2 * u + (j >> 1);
  else return w == 0 ? 2 * u + (j >> 1) : u;  // 3-bit: plane2 row, plane1 row
}

// Four fp16 pairs 1024 + q for the 8 codes lane group j takes from its
// word(s) of one column. Element order (pair p = elements 2p, 2p+1):
//  4-bit: slots (p, p + 4) of the word          -> k = 8j + {p, p+4}
//  8-bit: slots (0,1),(2,3) of word 0, then of 1 -> k = 8j + e
//  2/3-bit: slots (i0 + p, i0 + p + 8), i0 = 4 (j & 1), of the plane-2 word
//           -> k = 16 (j >> 1) + i0 + {p, p + 8}
template <int BITS>
__device__ __forceinline__ void decode8(uint32_t w0, uint32_t w1, int j, uint32_t (&b)[4]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int p = 0; p < 4; ++p) b[p] = ((w0 >> (4 * p)) & 0x000F000Fu) | kMagic1024x2;
  } else if constexpr (BITS == 8) {
    // byte permute: (byte0, 0x64, byte1, 0x64) = halves (1024 + q0, 1024 + q1)
    b[0] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
    b[1] = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
    b[2] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
    b[3] = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
  } else if constexpr (BITS == 2) {
    const uint32_t ws = w0 >> (8 * (j & 1));
#pragma unroll
    for (int p = 0; p < 4; ++p) b[p] = ((ws >> (2 * p)) & 0x00030003u) | kMagic1024x2;
  } else {
    // plane2 word w0 holds q >> 1 for 16 k; plane1 word w1 holds q & 1 for the
    // unit's 32 k. Gather the low bits of this word's slots 0-7 into bits 0-7
    // and of slots 8-15 into bits 16-23, so one shift serves both halves.
    const int base = 16 * (j >> 1);
    const uint32_t lo8 = (w1 >> base) & 0xFFu;
    const uint32_t hi8 = (w1 >> (base + 8)) & 0xFFu;
    const int i0 = 4 * (j & 1);
    const uint32_t ls = (lo8 | (hi8 << 16)) >> i0;
    const uint32_t hs = (w0 >> (2 * i0)) << 1;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      b[p] = ((hs >> (2 * p)) & 0x00060006u) | ((ls >> p) & 0x00010001u) | kMagic1024x2;
  }
}

__device__ __forceinline__ f16x8 pack8(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
  u32x4 v = {a0, a1, a2, a3};
  return __builtin_bit_cast(f16x8, v);
}

struct GemvArgs {
  const uint16_t* x;
  const uint32_t* qw;
  const uint32_t* qlo;
  const uint16_t* zeros;
  const uint16_t* scales;
  uint16_t* y;
  float* part;
  uint32_t* counters;
  int M, K, N;
  int upg;       // 32-row units per group
  int upg_log2;  // log2(upg) when upg is a power of two, else -1
  int units_per_block;
  int ksplit;
};

// Units (32 rows of K) per batch of loads issued together, bounded by the
// registers a wave may hold (128 with 16 waves per block).
template <int BITS, int VEC, int WAVES> constexpr int chunk_units() {
  return (Bits<BITS>::NW * VEC <= (WAVES >= 8 ? 2 : 4)) ? 8 : 4;
}

// Fp16 scale/zero values of a lane's VEC columns, as loaded.
template <int VEC> struct Halves;
template <> struct Halves<1> { typedef uint16_t T; };
template <> struct Halves<2> { typedef uint32_t T; };
template <> struct Halves<4> { typedef u32x2 T; };
template <int VEC>
__device__ __forceinline__ typename Halves<VEC>::T load_halves(const uint16_t* p) {
  return *reinterpret_cast<const typename Halves<VEC>::T*>(p);
}
template <int VEC>
__device__ __forceinline__ uint16_t half_at(typename Halves<VEC>::T h, int v) {
  if constexpr (VEC == 1) return h;
  else if constexpr (VEC == 2) return (uint16_t)(h >> (16 * v));
  else return (uint16_t)(h[v >> 1] >> (16 * (v & 1)));
}

// Raw activation bytes of one unit for lane group j: 16 halves' worth of
// registers, permuted into decode8's element order when used.
template <int BITS>
__device__ __forceinline__ u32x4 load_x_raw(const uint16_t* ubase, uint32_t off) {
  if constexpr (BITS == 4 || BITS == 8) {
    return *reinterpret_cast<const u32x4*>(ubase + off);
  } else {
    const u32x2 e = *reinterpret_cast<const u32x2*>(ubase + off);
    const u32x2 f = *reinterpret_cast<const u32x2*>(ubase + off + 8);
    return u32x4{e.x, e.y, f.x, f.y};
  }
}

// The A operand (x[m, 32u + k] for the 8 k of lane group j, in decode8's
// element order) from the raw registers.
template <int BITS>
__device__ __forceinline__ f16x8 x_operand(u32x4 d) {
  uint32_t a0, a1, a2, a3;
  if constexpr (BITS == 8) {
    a0 = d.x; a1 = d.y; a2 = d.z; a3 = d.w;
  } else {
    // 4-bit: d = x[0..7], pairs (k, k + 4); 2/3-bit: d = x[o..o+3], x[o+8..o+11], pairs (k, k + 8)
    const uint32_t lo0 = d.x, lo1 = d.y;
    const uint32_t hi0 = (BITS == 4) ? d.z : d.z, hi1 = (BITS == 4) ? d.w : d.w;
    a0 = (lo0 & 0xFFFFu) | (hi0 << 16);
    a1 = (lo0 >> 16) | (hi0 & 0xFFFF0000u);
    a2 = (lo1 & 0xFFFFu) | (hi1 << 16);
    a3 = (lo1 >> 16) | (hi1 & 0xFFFF0000u);
  }
  return pack8(a0, a1, a2, a3);
}

// Word-row offset of lane group j's first word of plane w within a unit, and
// the rows a unit spans in that plane.
template <int BITS>
__device__ __forceinline__ int lane_row(int j, int w) {
  if constexpr (BITS == 4) return j;
  else if constexpr (BITS == 8) return 2 * j + w;
  else if constexpr (BITS == 2) return j >> 1;
  else return w == 0 ? (j >> 1) : 0;
}
template <int BITS>
__device__ __forceinline__ int unit_rows(int w) {
  if constexpr (BITS == 4) return 4;
  else if constexpr (BITS == 8) return 8;
  else if constexpr (BITS == 2) return 2;
  else return w == 0 ? 2 : 1;
}

template <int BITS, int VEC, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(GemvArgs g) {
  constexpr int NW = Bits<BITS>::NW;
  constexpr int CH = chunk_units<BITS, VEC, WAVES>();
  constexpr int COLS = 16 * VEC;
  constexpr int THREADS = 64 * WAVES;
  __shared__ float red[WAVES][kMaxM][COLS];
  __shared__ int last_flag;

  const int lane = threadIdx.x & 63;
  // The wave index is the same for every lane of a wave; saying so keeps all
  // unit bookkeeping below in scalar registers and scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane >> 4;       // lane group: which 8 k of a unit
  const int cl = lane & 15;      // column group within the wave
  // Workgroups are dealt to the 8 XCDs round-robin by linear id, and each
  // XCD has its own L2. Narrow strips share 128-byte lines with their
  // neighbours, so each XCD is given a contiguous run of strips: a line is
  // then fetched into one L2 only.
  int strip = blockIdx.x;
  if (QMM_GEMV_XCD_REMAP && (gridDim.x & 7) == 0) strip = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int split = blockIdx.y;
  const int n0 = strip * COLS;
  const int nc = n0 + VEC * cl;  // first of this lane's VEC columns
  const bool col_ok = nc < g.N;
  const int ncc = col_ok ? nc : 0;  // clamped: every load below is in bounds
  // A-operand row of this lane. Rows >= M read row 0: those MFMA rows only
  // produce outputs that are never stored, so they need no zeroing.
  const int m = cl < g.M ? cl : 0;

  const int U = g.K / 32;
  const int ub0 = split * g.units_per_block;
  const int ub1 = min(U, ub0 + g.units_per_block);
  const int per_wave = (g.units_per_block + WAVES - 1) / WAVES;
  const int ua = min(ub1, ub0 + wave * per_wave);
  const int uz = min(ub1, ua + per_wave);

  // Per-lane parts of every address; the per-unit parts are uniform.
  uint32_t woff[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) woff[w] = (uint32_t)(lane_row<BITS>(j, w) * g.N + ncc);
  const uint32_t xoff = (uint32_t)(m * g.K) +
                        ((BITS == 4 || BITS == 8) ? 8 * j : 16 * (j >> 1) + 4 * (j & 1));

  f32x4 total[VEC], acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    total[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float sc[VEC];
  f16x2 zc[VEC];  // -(1024 + z) on the exact path, else -z (1024 removed separately)
#pragma unroll
  for (int v = 0; v < VEC; ++v) { sc[v] = 0.f; zc[v] = f16x2{0, 0}; }
  int zfast = 1;
  int cur_g = -1;

  for (int base = ua; base < uz; base += CH) {
    typename Vec<VEC>::T wv[CH][NW];
    u32x4 xr[CH];
    typename Halves<VEC>::T sr[CH], zr[CH];
    // Issue every load of the batch (indices clamped into range) before any
    // of them is used.
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int u = min(base + c, uz - 1);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t* plane = (BITS == 3 && w == 1) ? g.qlo : g.qw;
        const uint32_t* ubase = plane + (size_t)u * unit_rows<BITS>(w) * g.N;
        wv[c][w] = load_words<VEC>(ubase + woff[w]);
      }
      xr[c] = load_x_raw<BITS>(g.x + 32 * u, xoff);
      const int grp = g.upg_log2 >= 0 ? (u >> g.upg_log2) : u / g.upg;
      const size_t gofs = (size_t)grp * g.N;
      sr[c] = load_halves<VEC>(g.scales + gofs + ncc);
      zr[c] = load_halves<VEC>(g.zeros + gofs + ncc);
    }
    auto process = [&](auto fast_tag, int c) {
      constexpr bool FAST = decltype(fast_tag)::value;
      const f16x8 A = x_operand<BITS>(xr[c]);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        uint32_t b[4];
        decode8<BITS>(word_at<VEC>(wv[c][0], v), NW > 1 ? word_at<VEC>(wv[c][NW - 1], v) : 0u, j, b);
        uint32_t d[4];
        if constexpr (FAST) {
#pragma unroll
          for (int p = 0; p < 4; ++p) d[p] = as_u32(as_f16x2(b[p]) + zc[v]);
        } else {
          const f16x2 m1024 = f16x2{(f16)(-1024.f), (f16)(-1024.f)};
#pragma unroll
          for (int p = 0; p < 4; ++p) d[p] = as_u32((as_f16x2(b[p]) + m1024) + zc[v]);
        }
        acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pack8(d[0], d[1], d[2], d[3]), acc[v], 0, 0, 0);
      }
    };
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int u = base + c;
      if (u >= uz) break;  // scalar
      const int grp = g.upg_log2 >= 0 ? (u >> g.upg_log2) : u / g.upg;
      if (grp != cur_g) {  // scalar
        if (cur_g >= 0) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            total[v] += sc[v] * acc[v];
            acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        cur_g = grp;
        bool exact = true;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          sc[v] = half_bits_to_float(half_at<VEC>(sr[c], v));
          const uint16_t zb = half_at<VEC>(zr[c], v);
          const float z = half_bits_to_float(zb);
          exact = exact && (z == __builtin_rintf(z)) && (__builtin_fabsf(z) <= 1024.f);
          const f16 zh = __builtin_bit_cast(f16, zb);
          zc[v] = f16x2{zh, zh};
        }
        zfast = __builtin_amdgcn_readfirstlane(__all(exact));
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          // exact when zfast: integer zero point, |z| <= 1024
          const f16 t = zfast ? (f16)((f16)(-1024.f) - zc[v].x) : (f16)(-zc[v].x);
          zc[v] = f16x2{t, t};
        }
      }
      if (zfast) process(std::integral_constant<bool, true>{}, c);
      else process(std::integral_constant<bool, false>{}, c);
    }
  }
  if (cur_g >= 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) total[v] += sc[v] * acc[v];
  }

  // D layout: lane holds rows 4 j + i (i < 4) of column VEC * cl + v.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * j + i;
    if (row < g.M) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) red[wave][row][VEC * cl + v] = total[v][i];
    }
  }
  __syncthreads();

  // Waves of the block are summed in wave order.
  const int entries = g.M * COLS;
  if (g.ksplit == 1) {
    for (int e = threadIdx.x; e < entries; e += THREADS) {
      const int row = e / COLS, col = e - row * COLS;
      if (n0 + col < g.N) {
        float s = red[0][row][col];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) s += red[w][row][col];
        g.y[(size_t)row * g.N + n0 + col] = __builtin_bit_cast(uint16_t, (f16)s);
      }
    }
    return;
  }

  // Blocks along K hand over through the workspace. Partial sums are written
  // and read with device-scope atomic accesses, which go to the
  // device-coherent level of the memory hierarchy rather than an XCD's own
  // L2; each thread waits until its stores are acknowledged before the block
  // takes its ticket, so the last block to arrive sees every partial.
  float* mypart = g.part + (size_t)split * g.M * g.N;
  for (int e = threadIdx.x; e < entries; e += THREADS) {
    const int row = e / COLS, col = e - row * COLS;
    if (n0 + col < g.N) {
      float s = red[0][row][col];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) s += red[w][row][col];
      __hip_atomic_store(mypart + (size_t)row * g.N + n0 + col, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): stores acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&g.counters[strip], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == (uint32_t)(g.ksplit - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  for (int e = threadIdx.x; e < entries; e += THREADS) {
    const int row = e / COLS, col = e - row * COLS;
    if (n0 + col < g.N) {
      const size_t off = (size_t)row * g.N + n0 + col;
      // All partials are requested before any is added (one round trip), then
      // summed in split order.
      float pv[kMaxSplit];
#pragma unroll
      for (int sp = 0; sp < kMaxSplit; ++sp) {
        const int spc = min(sp, g.ksplit - 1);
        pv[sp] = __hip_atomic_load(g.part + (size_t)spc * g.M * g.N + off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      float s = pv[0];
#pragma unroll
      for (int sp = 1; sp < kMaxSplit; ++sp) s += (sp < g.ksplit) ? pv[sp] : 0.f;
      g.y[off] = __builtin_bit_cast(uint16_t, (f16)s);
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(&g.counters[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, int VEC, int WAVES>
hipError_t launch_typed(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  dim3 grid(p.nstrips, p.ksplit);
  gemv_kernel<BITS, VEC, WAVES><<<grid, 64 * WAVES, 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if (p.vec == 1) return p.waves == 16 ? launch_typed<BITS, 1, 16>(p, a, s) : launch_typed<BITS, 1, 8>(p, a, s);
  if (p.waves == 16) return p.vec == 2 ? launch_typed<BITS, 2, 16>(p, a, s) : launch_typed<BITS, 4, 16>(p, a, s);
  if (p.waves == 8) return p.vec == 2 ? launch_typed<BITS, 2, 8>(p, a, s) : launch_typed<BITS, 4, 8>(p, a, s);
  return p.vec == 2 ? launch_typed<BITS, 2, 4>(p, a, s) : launch_typed<BITS, 4, 4>(p, a, s);
}

}  // namespace

GemvPlan gemv_plan(int M, int K, int N, int bits, int group_size) {
  GemvPlan p{};
  // Narrowest column strip whose blocks fit in one round on the 256 CUs
  // (16, 32 or 64 columns per wave). Every block then covers a strip with
  // 16 waves splitting K; blocks along K are added only when the strips
  // alone leave too few waves in flight.
  int vec = 4;
  if ((N + 15) / 16 <= kCUs) vec = 1;
  else if ((N + 31) / 32 <= kCUs) vec = 2;
  if (QMM_GEMV_VEC != 0) vec = QMM_GEMV_VEC;
  p.vec = vec;
  p.strip_cols = 16 * vec;
  p.nstrips = (N + p.strip_cols - 1) / p.strip_cols;
  const int U = K / 32;
  // 16 waves per block, except where two words per lane per unit (3-bit,
  // 8-bit) at 4 columns per lane need more registers than 16 waves allow.
  p.waves = (vec == 4 && (bits == 3 || bits == 8)) ? 8 : 16;
  if (QMM_GEMV_WAVES != 0) p.waves = QMM_GEMV_WAVES;
  const long long per_split = (long long)p.nstrips * p.waves;
  int ks = (int)((QMM_GEMV_TARGET_WAVES + per_split - 1) / per_split);
  int max_ks = U / p.waves;  // at least one unit per wave
  max_ks = max_ks < 1 ? 1 : (max_ks > kMaxSplit ? kMaxSplit : max_ks);
  ks = ks < 1 ? 1 : (ks > max_ks ? max_ks : ks);
  p.upg = group_rows(K, group_size) / 32;
  p.upg_log2 = -1;
  for (int l = 0; l < 31; ++l)
    if ((1 << l) == p.upg) p.upg_log2 = l;
  p.units_per_block = (U + ks - 1) / ks;
  p.ksplit = (U + p.units_per_block - 1) / p.units_per_block;
  if (p.ksplit > 1) {
    p.counters_bytes = kCounterHeaderBytes;
    p.workspace_bytes = p.counters_bytes + (size_t)p.ksplit * M * N * sizeof(float);
  }
  return p;
}

hipError_t launch_gemv(const GemvPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                       const uint32_t* qlo, const uint16_t* zeros, const uint16_t* scales, int N,
                       int bits, int group_size, uint16_t* y, void* workspace, hipStream_t s) {
  GemvArgs a;
  a.x = x;
  a.qw = qw;
  a.qlo = qlo;
  a.zeros = zeros;
  a.scales = scales;
  a.y = y;
  a.counters = p.ksplit > 1 ? static_cast<uint32_t*>(workspace) : nullptr;
  a.part = p.ksplit > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + p.counters_bytes) : nullptr;
  a.M = M;
  a.K = K;
  a.N = N;
  a.upg = p.upg;
  a.upg_log2 = p.upg_log2;
  a.units_per_block = p.units_per_block;
  a.ksplit = p.ksplit;
  switch (bits) {
    case 2: return launch_bits<2>(p, a, s);
    case 3: return launch_bits<3>(p, a, s);
    case 4: return launch_bits<4>(p, a, s);
    case 8: return launch_bits<8>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
