// Decode product internals shared by the split kernel (gemv.hip) and the
// wave-local kernels (gemv_wave.h, one translation unit per code width):
// the kernel arguments, the code layout per width, decoding into fp16 pairs
// and buffer loads.
#pragma once

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
#ifndef QMM_GEMV_WAVE_X
#define QMM_GEMV_WAVE_X 1  // wave kernel: waves stage their own activations (0: the block, one barrier)
#endif
#ifndef QMM_GEMV_XSUM_LDS
#define QMM_GEMV_XSUM_LDS 1  // wave kernel, one row with block staging: sums of x per group from the staged slots
#endif
#ifndef QMM_GEMV_SZ_SHARE
#define QMM_GEMV_SZ_SHARE 1  // wave kernel, several rows: lane groups request one group's scales / zero points each and share them
#endif
#ifndef QMM_GEMV_XCD_REMAP
#define QMM_GEMV_XCD_REMAP 1
#endif
#ifndef QMM_GEMV_ONE_XCD
#define QMM_GEMV_ONE_XCD 1  // wave kernel: strips that fit on one XCD's CUs all run there
#endif

namespace qmm {

struct GemvArgs {
  const uint16_t* x;
  const uint32_t* qw;
  const uint32_t* qlo;
  const uint16_t* zeros;
  const uint16_t* scales;
  const uint16_t* bias;  // (N,) or null
  uint16_t* y;
  float* part;
  uint32_t* counters;
  int M, K, N;
  int upg;       // 32-row units per group
  int upg_log2;  // log2(upg) when upg is a power of two, else -1
  int units_per_block;
  int ksplit;
  int ubp_log2;  // log2 of the activation slots per row and lane group (>= units_per_block)
  int gp_log2;   // log2 of the rows of scales / zero points staged per block
  int xcd_log2;  // log2 of the XCD count when that is a power of two dividing the grid's x size, else -1
  int gl;        // wave kernel: log2 of the units per group (30 for one group over all of K)
  int strips;    // packed words in the 16-column strip-major layout (else K-major)
  int one_xcd;   // wave kernel: the XCD count when the grid is that many times the strips and only XCD 0's blocks work, else 0
};

namespace {

// Words per lane per unit and column: 4-bit 1 row, 8-bit 2 rows, 2-bit 1 row
// (two lane groups share it), 3-bit one word of each plane.
template <int BITS> struct Bits;
template <> struct Bits<4> { static constexpr int NW = 1; };
template <> struct Bits<8> { static constexpr int NW = 2; };
template <> struct Bits<2> { static constexpr int NW = 1; };
template <> struct Bits<3> { static constexpr int NW = 2; };
template <> struct Bits<1> { static constexpr int NW = 1; };

template <int VEC> struct Vec;
template <> struct Vec<1> { typedef uint32_t T; };
template <> struct Vec<2> { typedef u32x2 T; };
template <> struct Vec<4> { typedef u32x4 T; };

template <int VEC>
__device__ __forceinline__ uint32_t word_at(typename Vec<VEC>::T w, int v) {
  if constexpr (VEC == 1) return w;
  else return w[v];
}

// (w & m) | (c & ~m). With m and c held in registers (below) this is one
// bitfield insert (v_bfi_b32) instead of an AND and an OR with literals.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t w, uint32_t c) { return (w & m) | (c & ~m); }

// Masks of decode8, made once per kernel: the empty asm statements keep them
// in registers (a vector register per mask, the magic 1024.0 pair in a scalar
// one) instead of being folded back into literals.
template <int BITS> struct DecodeMasks {
  uint32_t m[4];
  uint32_t magic;
};
// SUB: the codes become fp16 subnormals (exponent field 0, value 2^e q 2^-24)
// instead of 1024 + 2^e q: the same inserts into a zero word, which the
// compiler reduces to ANDs.
template <int BITS, bool SUB = false> __device__ __forceinline__ DecodeMasks<BITS> decode_masks() {
  DecodeMasks<BITS> d;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    d.m[p] = BITS == 4 ? (p & 1 ? 0x00F000F0u : 0x000F000Fu)
           : BITS == 2 ? (p & 1 ? 0x000C000Cu : 0x00030003u)
           : (BITS == 3 && SUB) ? (0x00060006u << (2 * p - (p > 0 ? 1 : 0)))  // pair p's 2-bit plane: bits 2p, 2p + 1 (pair 0: 1, 2)
           : BITS == 3 ? (p & 1 ? 0x00020002u : 0x000C000Cu)  // 2-bit plane at bits 2-3, 1-bit plane at bit 1
           : BITS == 1 ? ((1u << p) | (1u << (20 + p))) : 0u;
    if (BITS == 1 || (BITS == 3 && SUB) || ((BITS == 2 || BITS == 3 || BITS == 4) && p < 2)) asm("" : "+v"(d.m[p]));
  }
  d.magic = SUB ? 0u : kMagic1024x2;
  if (!SUB) asm("" : "+s"(d.magic));
  return d;
}

// Place of a code in the fp16 mantissa after decode8: half `hi` of pair p
// holds 1024 + 2^e q with e = code_exp(p, hi).
template <int BITS> __host__ __device__ constexpr int code_exp(int p, int hi) {
  return BITS == 4 ? 4 * (p & 1) : BITS == 2 ? 2 * (p & 1) : BITS == 1 ? p + 4 * hi : BITS == 3 ? 1 : 0;
}
// The same for the subnormal form (decode8 with SUB): 3-bit pair p sits at
// e = 0, 1, 3, 5, where its 2-bit plane bits already are (no shift for pairs
// 1-3); 2-bit pair p at e = 2p, where it is in the word (no shift); every
// other width as above.
template <int BITS> __host__ __device__ constexpr int code_exp_sub(int p, int hi) {
  return BITS == 3 ? (p == 0 ? 0 : 2 * p - 1) : BITS == 2 ? 2 * p : code_exp<BITS>(p, hi);
}

// Four fp16 pairs 1024 + 2^e q for the 8 codes lane group j takes from its
// word(s) of one column. Element order (pair p = elements 2p, 2p+1):
//  4-bit: slots (p, p + 4) of the word          -> k = 8j + {p, p+4}
//  1-bit: slots (8j + p, 8j + p + 4) of the word -> k = 8j + {p, p+4}
//  8-bit: slots (0,1),(2,3) of word 0, then of 1 -> k = 8j + e
//  2/3-bit: slots (i0 + p, i0 + p + 8), i0 = 4 (j & 1), of the plane-2 word
//           -> k = 16 (j >> 1) + i0 + {p, p + 8}
// 4-bit: odd pairs are masked 4 places up (one shift for all four pairs);
// 2-bit: odd pairs 2 places up (two shifts); 1-bit: byte j is copied into
// both halves and pair p masked at bit p of the low half and bit 4 + p of the
// high half; 3-bit: q >> 1 (2-bit plane) goes to bits 2-3 and q & 1 (1-bit
// plane, its bytes of this lane group copied into both halves) to bit 1, so
// each half is 1024 + 2q.
// With SUB (decode_masks<BITS, true>) the codes are fp16 subnormals: half
// `hi` of pair p is 2^e q 2^-24 exactly, with e = code_exp_sub(p, hi) (the
// same places for 1-, 4- and 8-bit codes; 2- and 3-bit codes stay where their
// bits are in the words). The element order is the same in both forms.
template <int BITS, bool SUB = false>
__device__ __forceinline__ void decode8(uint32_t w0, uint32_t w1, int j, const DecodeMasks<BITS>& dm,
                                        uint32_t (&b)[4]) {
  const uint32_t magic = SUB ? 0u : dm.magic;
  const uint32_t mag8 = SUB ? 0u : 0x64646464u;
  if constexpr (BITS == 4) {
    const uint32_t t = w0 >> 8;
    b[0] = bfi(dm.m[0], w0, magic);
    b[1] = bfi(dm.m[1], w0, magic);
    b[2] = bfi(dm.m[0], t, magic);
    b[3] = bfi(dm.m[1], t, magic);
  } else if constexpr (BITS == 1) {
    // bytes (j, 0, j, 0) of the word: 0x0C selects a zero byte
    const uint32_t t = __builtin_amdgcn_perm(0u, w0, (uint32_t)j | 0x0C000C00u | ((uint32_t)j << 16));
#pragma unroll
    for (int p = 0; p < 4; ++p) b[p] = bfi(dm.m[p], t, magic);
  } else if constexpr (BITS == 8) {
    // byte permute: (byte0, 0x64, byte1, 0x64) = halves (1024 + q0, 1024 + q1)
    // (with SUB zero bytes in place of 0x64: halves q0 2^-24, q1 2^-24)
    b[0] = __builtin_amdgcn_perm(mag8, w0, 0x04010400u);
    b[1] = __builtin_amdgcn_perm(mag8, w0, 0x04030402u);
    b[2] = __builtin_amdgcn_perm(mag8, w1, 0x04010400u);
    b[3] = __builtin_amdgcn_perm(mag8, w1, 0x04030402u);
  } else if constexpr (BITS == 2) {
    const uint32_t ws = w0 >> (8 * (j & 1));
    if constexpr (SUB) {
      // subnormal form: pair p stays at bits 2p, 2p + 1 of each half (e = 2p)
#pragma unroll
      for (int p = 0; p < 4; ++p) b[p] = ws & (0x00030003u << (2 * p));
    } else {
      const uint32_t t = ws >> 4;
      b[0] = bfi(dm.m[0], ws, magic);
      b[1] = bfi(dm.m[1], ws, magic);
      b[2] = bfi(dm.m[0], t, magic);
      b[3] = bfi(dm.m[1], t, magic);
    }
  } else {
    // plane2 word w0 holds q >> 1 for 16 k (slot i0 + p of pair p at bits
    // 2 (i0 + p) and 2 (i0 + p) + 16); plane1 word w1 holds q & 1 for the
    // unit's 32 k (k = 16 (j >> 1) + i0 + p at that bit, and 8 more for the
    // high half). After the shifts below, pair p's planes sit at bits 2p of
    // hs and p of ls (low half) and 16 more (high half).
    const int i0 = 4 * (j & 1);
    const uint32_t hs = w0 >> (2 * i0);
    const uint32_t t = w1 >> (16 * (j >> 1) + i0);
    const uint32_t ls = __builtin_amdgcn_perm(0u, t, 0x0C010C00u);  // bytes (0, -, 1, -) of t
    if constexpr (SUB) {
      // Subnormal form, pair p at e = code_exp_sub: (2 h + l) 2^e with the
      // 2-bit plane where it already is (bits 2p, 2p + 1; pair 0 one place up)
      // and the low bit just below it.
      b[0] = bfi(dm.m[0], hs << 1, ls & 0x00010001u);
      b[1] = bfi(dm.m[1], hs, ls & 0x00020002u);
      b[2] = bfi(dm.m[2], hs, (ls << 1) & 0x00080008u);
      b[3] = bfi(dm.m[3], hs, (ls << 2) & 0x00200020u);
    } else {
      b[0] = bfi(dm.m[0], hs << 2, bfi(dm.m[1], ls << 1, magic));
      b[1] = bfi(dm.m[0], hs, bfi(dm.m[1], ls, magic));
      b[2] = bfi(dm.m[0], hs >> 2, bfi(dm.m[1], ls >> 1, magic));
      b[3] = bfi(dm.m[0], hs >> 4, bfi(dm.m[1], ls >> 2, magic));
    }
  }
}

__device__ __forceinline__ f16x8 pack8(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3) {
  u32x4 v = {a0, a1, a2, a3};
  return __builtin_bit_cast(f16x8, v);
}



// Units (32 rows of K) per batch of loads issued together, bounded by the
// registers a wave may hold (128 with 16 waves per block).
template <int BITS, int VEC, int WAVES> constexpr int chunk_units() {
  return (Bits<BITS>::NW * VEC <= (WAVES >= 8 ? 2 : 4)) ? 8 : 4;
}

// Pair classes: pairs whose codes sit at the same mantissa places.
template <int BITS> constexpr int kPairClasses = BITS == 1 ? 4 : ((BITS == 2 || BITS == 4) ? 2 : 1);
template <int BITS> __device__ __forceinline__ constexpr int pair_class(int p) {
  return BITS == 1 ? p : ((BITS == 2 || BITS == 4) ? (p & 1) : 0);
}
// 2^-e per half of pair p.
template <int BITS> __device__ __forceinline__ f16x2 pair_scale(int p) {
  return f16x2{(f16)(1.0f / (float)(1 << code_exp<BITS>(p, 0))), (f16)(1.0f / (float)(1 << code_exp<BITS>(p, 1)))};
}
// h 2^-e + c, one packed operation (an add where e is 0 in both halves).
template <int BITS> __device__ __forceinline__ f16x2 scale_add(int p, f16x2 h, f16x2 c) {
  if (code_exp<BITS>(p, 0) == 0 && code_exp<BITS>(p, 1) == 0) return h + c;
  return __builtin_elementwise_fma(h, pair_scale<BITS>(p), c);
}

// First k (within a unit) of the activations lane group j feeds: 8 consecutive
// k for 4- and 8-bit codes; for 2- and 3-bit codes two runs of 4, 8 apart.
template <int BITS> __device__ __forceinline__ int x_first(int j) {
  return (BITS == 1 || BITS == 4 || BITS == 8) ? 8 * j : 16 * (j >> 1) + 4 * (j & 1);
}

// A raw buffer resource over `bytes` bytes at p (out-of-range reads return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;  // buffer-load cache policy: streamed data

template <int VEC>
__device__ __forceinline__ typename Vec<VEC>::T load_words(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (VEC == 1) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal);
  else if constexpr (VEC == 2) return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNonTemporal);
  else return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal);
}

// Raw activation bytes of one (row, unit, lane group) slot: 8 halves.
template <int BITS>
__device__ __forceinline__ u32x4 load_x_slot(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  if constexpr (BITS == 1 || BITS == 4 || BITS == 8) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  } else {
    const u32x2 e = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
    const u32x2 f = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off + 16, 0, 0);
    return u32x4{e.x, e.y, f.x, f.y};
  }
}

// The A operand (x[m, 32u + k] for the 8 k of lane group j, in decode8's
// element order) from the raw registers.
template <int BITS>
__device__ __forceinline__ u32x4 x_operand(u32x4 d) {
  if constexpr (BITS == 8) {
    return d;
  } else {
    // 1/4-bit: d = x[0..7], pairs (k, k + 4); 2/3-bit: d = x[o..o+3], x[o+8..o+11], pairs (k, k + 8)
    const uint32_t lo0 = d.x, lo1 = d.y, hi0 = d.z, hi1 = d.w;
    return u32x4{__builtin_amdgcn_perm(hi0, lo0, 0x05040100u), __builtin_amdgcn_perm(hi0, lo0, 0x07060302u),
                 __builtin_amdgcn_perm(hi1, lo1, 0x05040100u), __builtin_amdgcn_perm(hi1, lo1, 0x07060302u)};
  }
}

// Word-row offset of lane group j's first word of plane w within a unit, and
// the rows a unit spans in that plane.
template <int BITS>
__device__ __forceinline__ int lane_row(int j, int w) {
  if constexpr (BITS == 1) return 0;
  else if constexpr (BITS == 4) return j;
  else if constexpr (BITS == 8) return 2 * j + w;
  else if constexpr (BITS == 2) return j >> 1;
  else return w == 0 ? (j >> 1) : 0;
}
template <int BITS>
__device__ __forceinline__ int unit_rows(int w) {
  if constexpr (BITS == 1) return 1;
  else if constexpr (BITS == 4) return 4;
  else if constexpr (BITS == 8) return 8;
  else if constexpr (BITS == 2) return 2;
  else return w == 0 ? 2 : 1;
}

// Workgroups are dealt to the XCDs round-robin by linear id, and each XCD has
// its own L2. Narrow strips share 128-byte lines with their neighbours, so
// each XCD is given a contiguous run of strips: a line is then fetched into
// one L2 only. The host passes log2 of the XCD count when that is a power of
// two dividing the number of strips, else -1 (identity).
__device__ __forceinline__ int xcd_strip(int b, int nb, int xcd_log2) {
  if (!QMM_GEMV_XCD_REMAP || xcd_log2 < 0) return b;
  return (b & ((1 << xcd_log2) - 1)) * (nb >> xcd_log2) + (b >> xcd_log2);
}

}  // namespace
}  // namespace qmm
