// Prefill product y = x @ dequant(W) for any M on gfx950's matrix cores.
//
// What is computed is the dense product of x with the dequantized weight
// (dashq_kernel.py, TritonQuantLinear.forward batched path and
// dequantize_weight; GPTQModel-Compatible Triton Kernel README, overview: the
// dequantization is fused into the product instead of materialising W).
//
// Design:
//  * Block tile 256 x 256, K in slabs of 64; 8 waves in a 2 (M) x 4 (N)
//    arrangement, each wave a 128 x 64 sub-tile of 4 x 2
//    V_MFMA_F32_32X32X16_F16 accumulators (128 fp32 registers per lane).
//    Products too small to give every CU such a tile take 128 x 128 or
//    64 x 64 tiles of 4 waves (the README's own benchmark shapes are of this
//    kind).
//  * Activations go straight from memory into LDS (buffer loads with the
//    LDS destination, no registers), three slabs rotating, each requested two
//    slabs before its first read; rows are unpadded and their 16-byte chunks
//    XOR-swizzled so the fragment reads of a wave spread over all banks. One
//    barrier per slab publishes the next slab.
//  * Weights never touch LDS. Each lane loads exactly the packed words of its
//    own B fragments with buffer loads two slabs ahead; a wave's two column
//    tiles take interleaved columns, so one 8-byte load brings a lane the
//    words of both (the 32 lanes of a half wave read 256 contiguous bytes).
//  * Software pipelining: while a 16-k step's MFMAs run, the next step's A
//    fragments are read from LDS and its weight words dequantized, and the
//    compiler is asked to interleave these with the MFMAs one by one.
//  * Dequantization: codes are placed in the mantissa of 1024.0 (a byte
//    permute, or a field extract and masked inserts) and the zero point is
//    subtracted in fp16. With one group per column, one packed add of
//    c = -(1024 + z) rounded to fp16 subtracts z rounded to an integer (for
//    |z| < 1024; exactly); the remainder (zero for integer zero points) is
//    removed in the epilogue with the row sums of x, and the scale is applied
//    to the fp32 accumulator. With smaller groups each half is
//    (q - z) * scale in fp16 (one rounding of an exact difference).
//  * Register sets of two slabs in flight and of the fragments of two steps
//    are indexed by compile-time parity (two slabs per loop iteration), so no
//    registers are copied between sets.
//  * The epilogue stores straight from the accumulators: a lane's two
//    paired columns are adjacent, one 4-byte store each.
//  * Each XCD (own L2 each) works on a contiguous range of tiles,
//    walked in groups of row tiles so that the blocks in flight on it share
//    weight and activation panels.
#include <type_traits>

#include "common.h"

namespace qmm {
namespace {

constexpr int BK = 64;

struct GemmArgs {
  const uint16_t* x;
  const uint32_t* qw;
  const uint32_t* qlo;
  const uint16_t* zeros;
  const uint16_t* scales;
  const uint16_t* bias;  // (N,) or null
  uint16_t* y;
  int M, K, N;
  int upg;       // 32-row units per group
  int upg_log2;  // log2(upg) if a power of two, else -1
  int mblocks, nblocks;
  int xcds;      // XCDs of the device; blocks are dealt to them round-robin
  int cus;       // compute units of the device
  int strips;    // packed words in the 16-column strip-major layout (else K-major)
};

// Words one lane needs for one 32-column tile and one 16-k step: a 32 x 32 x 16
// MFMA B fragment gives lane l the 8 consecutive k of chunk l / 32 of the
// step, for column l % 32. NW words of the main plane, NL of the 1-bit plane
// (3-bit codes).
template <int BITS> struct Frag;
template <> struct Frag<8> { static constexpr int NW = 2, NL = 0, EPS = 4; };
template <> struct Frag<4> { static constexpr int NW = 1, NL = 0, EPS = 8; };
template <> struct Frag<2> { static constexpr int NW = 1, NL = 0, EPS = 16; };
template <> struct Frag<3> { static constexpr int NW = 1, NL = 1, EPS = 16; };
template <> struct Frag<1> { static constexpr int NW = 1, NL = 0, EPS = 32; };

// Word row (within the plane) of word w of k-step s of slab ks, for lane
// chunk kc.
template <int BITS>
__device__ __forceinline__ int frag_row(int ks, int s, int kc, int w) {
  if constexpr (BITS == 8) return ks * 16 + 4 * s + 2 * kc + w;
  else if constexpr (BITS == 4) return ks * 8 + 2 * s + kc;
  else if constexpr (BITS == 1) return ks * 2 + (s >> 1);  // 32 codes per word: two steps
  else return ks * 4 + s;  // 2-bit and the 2-bit plane of 3-bit codes
}

// Four fp16 pairs 1024 + q (pair p = codes 2p, 2p + 1 of the lane's 8 k) from
// the fragment's words. kc selects the lane's half of a 16-code word; s the
// 16-k step within the 32 codes of a 1-bit plane word.
template <int BITS>
__device__ __forceinline__ void frag_codes(const uint32_t* w, const uint32_t* l, int kc, int s, uint32_t (&h)[4]) {
  if constexpr (BITS == 8) {
    // byte permute: (byte, 0x64, byte, 0x64) = halves 1024 + q
    h[0] = __builtin_amdgcn_perm(0x64646464u, w[0], 0x04010400u);
    h[1] = __builtin_amdgcn_perm(0x64646464u, w[0], 0x04030402u);
    h[2] = __builtin_amdgcn_perm(0x64646464u, w[1], 0x04010400u);
    h[3] = __builtin_amdgcn_perm(0x64646464u, w[1], 0x04030402u);
  } else if constexpr (BITS == 4) {
    // Byte p of w in the low half and byte p of w >> 4 in the high half put
    // codes 2p and 2p + 1 each in the low nibble of a half; the mask is held
    // in a register so that the AND and the OR with 1024.0 are one
    // v_and_or_b32 (an instruction of this form takes one literal).
    const uint32_t w4 = w[0] >> 4;
    uint32_t m = 0x000F000Fu;
    asm("" : "+v"(m));
#pragma unroll
    for (int p = 0; p < 4; ++p)
      h[p] = (__builtin_amdgcn_perm(w4, w[0], 0x0C040C00u | (uint32_t)p | ((uint32_t)p << 16)) & m) | kMagic1024x2;
  } else {
    // The lane's 8 codes come from one extract per plane. Doubling a field
    // (x | x << 15, or x << 1 | x << 15 for the 2-bit plane of 3-bit codes)
    // puts code 2p + 1's bits 16 places above code 2p's once shifted right
    // by p fields, so one or two bit-field inserts per pair into 1024.0 give
    // both halves 1024 + q.
    if constexpr (BITS == 3) {
      const uint32_t u = __builtin_amdgcn_ubfe(w[0], 16 * kc, 16);
      const uint32_t v = __builtin_amdgcn_ubfe(l[0], 16 * (s & 1) + 8 * kc, 8);
      const uint32_t bh = (u << 1) | (u << 15), bl = v | (v << 15);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = ((bl >> (2 * p)) & 0x00010001u) | (kMagic1024x2 & ~0x00010001u);
        h[p] = ((bh >> (4 * p)) & 0x00060006u) | (lo & ~0x00060006u);
      }
    } else {
      // 1024.0 has zeros under the mask, so an insert is (x & m) | 1024.0;
      // the mask is held in a register so that it is one v_and_or_b32.
      uint32_t m = BITS == 1 ? 0x00010001u : 0x00030003u;
      asm("" : "+v"(m));
      const uint32_t x = BITS == 1 ? __builtin_amdgcn_ubfe(w[0], 16 * (s & 1) + 8 * kc, 8)
                                   : __builtin_amdgcn_ubfe(w[0], 16 * kc, 16);
      const uint32_t b = BITS == 1 ? x | (x << 15) : x | (x << 14);
#pragma unroll
      for (int p = 0; p < 4; ++p) h[p] = ((b >> ((BITS == 1 ? 2 : 4) * p)) & m) | kMagic1024x2;
    }
  }
}

// Tile (mb, nb) of block pid. Dispatch places block ids round-robin on the 8
// XCDs (each with its own L2), so each XCD is given a contiguous range of
// tiles. When that range is made of whole columns of row tiles, it is walked
// in groups of 4 (or 2) row tiles across its columns, so that the blocks in
// flight on an XCD share fewer activation panels and more weight panels:
// about 15% fewer L2 misses per slab than one whole column after another.
__device__ __forceinline__ void tile_of_block(int pid, int mblocks, int nblocks, int xcds, int& mb, int& nb) {
  const int n = mblocks * nblocks;
  if (xcds <= 1 || n % xcds != 0) {
    nb = pid / mblocks;
    mb = pid - nb * mblocks;
    return;
  }
  const int per = n / xcds, x = pid % xcds, li = pid / xcds;
  const int rg = mblocks % 4 == 0 ? 4 : (mblocks % 2 == 0 ? 2 : 1);
  if (rg > 1 && per % mblocks == 0) {
    const int ncx = per / mblocks;  // columns of the XCD's range
    const int gi = li / (rg * ncx), rem = li - gi * (rg * ncx);
    nb = x * ncx + rem / rg;
    mb = gi * rg + rem % rg;
    return;
  }
  const int tile = x * per + li;
  nb = tile / mblocks;
  mb = tile - nb * mblocks;
}

// A raw buffer resource over `bytes` bytes at p (out-of-range reads return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
// Wait until at most n vector-memory operations of this wave are in flight
// (s_waitcnt's vmcnt field, expcnt and lgkmcnt left unconstrained).
#ifndef QMM_GEMM_SPREAD
#define QMM_GEMM_SPREAD 1
#endif
#ifndef QMM_GEMM_NBUF4
#define QMM_GEMM_NBUF4 1
#endif
#define QMM_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// A 16-byte-per-lane load from a buffer straight into LDS: lane l's bytes
// land at lds_addr + 16 l (lds_addr wave-uniform). Written as one asm block
// because the compiler, seeing such a store through the builtin, would make
// every later LDS read wait for it; completion is instead awaited with an
// explicit vmcnt before the barrier that publishes the slab. No vector
// register is written; m0 carries the LDS address and is restored after.
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Cache policy of the weight loads: the scope bit only (no non-temporal
// hint), which measured fastest; a weight panel is reused by the row tiles
// that run beside each other on one XCD.
constexpr int kWeightPolicy = 1;


// Block tile BM x BN = (32 TM WM) x (32 TN WN), computed by KG groups of
// WM x WN waves, each wave TM x TN MFMA tiles of 32 x 32. Group j takes the
// 64-k slabs j, j + KG, j + 2 KG, ... with LDS buffers of its own; the groups'
// fp32 sums are added in group order at the end.
// BF: bf16 data (x, scales, zero points, bias, y); dequantized codes are then
// formed in fp32 and rounded once to bf16 for the bf16 matrix-core form.
// ZM, how zero points and scales vary along K: 2, one group per column (the
// scale is applied to the fp32 sums); 1, groups of whole 64-k slabs (one
// row per slab); 0, groups of 32-k units (one row per unit).
template <int BITS, int ZM, bool KTAIL, int WM, int WN, int TM, int TN, int KG, bool BF>
__global__ __launch_bounds__(64 * WM * WN * KG, 1) void gemm_kernel(GemmArgs g) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  constexpr int GW = WM * WN;  // waves per group
  constexpr int ACC = TM * TN * 16;  // accumulators per lane
  // Each group's three activation buffers; then, reusing them, the other
  // groups' partial sums.
  // Activation slab buffers per group: four where they fit the LDS (with the
  // spread loads, the fourth lengthens how far ahead a slab's last quarter is
  // requested from 5 steps to 9), else three.
  constexpr int NBUF = (QMM_GEMM_NBUF4 && KG * 4 * BM * BK * 2 + BM * 4 <= 160 * 1024) ? 4 : 3;
  constexpr int kLdsHalves = cmax(KG * NBUF * BM * BK, (KG - 1) * GW * ACC * 64 * 2);
  __shared__ __attribute__((aligned(16))) f16 lds[kLdsHalves];
  __shared__ float rsum[BM];  // row sums of x, for zero points that are not integers
  constexpr int GT = 64 * GW;  // threads per group
  constexpr int THREADS = GT * KG;
  constexpr int CQ = BM * BK * 2 / 1024 / GW;  // 1 KiB activation loads per wave per slab
  static_assert(CQ >= 1 && CQ * GW * 1024 == BM * BK * 2, "slab must split into 1 KiB loads per wave");
  constexpr int NW = Frag<BITS>::NW, NL = Frag<BITS>::NL;
  constexpr bool POST_SCALE = ZM == 2;
  constexpr int NG = ZM == 0 ? 2 : 1;  // rows of zero points / scales per slab
  // Activation loads of a slab spread over its four steps (one 1 KiB load
  // per wave and step) instead of four in one step, where they fill the
  // texture unit's command queue and hold back the next instructions.
  constexpr bool SPREAD = QMM_GEMM_SPREAD && CQ == 4;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / GW;        // K group
  const int gwave = wave - kg * GW;  // wave within the group
  const int wm = gwave / WN, wn = gwave % WN;
  const int kc = lane >> 5;  // k chunk of the lane in a fragment

  int mb, nb;
  tile_of_block(blockIdx.x, g.mblocks, g.nblocks, g.xcds, mb, nb);
  const int m0 = mb * BM, n0 = nb * BN;
  const int nk = (int)(((uint32_t)g.K + BK - 1) / BK);
  const int ni = (nk + KG - 1) / KG;  // slabs per group (the last ones may pad)
  auto gslab = [&](int i) { return kg + KG * i; };  // global slab of the group's i-th

  // Buffer resources: every global load below is a 32-bit per-lane offset
  // plus a scalar offset, which keeps address arithmetic out of the vector
  // registers.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.x, (size_t)g.M * g.K * 2);
  const int wrs = plane_row_stride(g.N, g.strips);
  const long long wcols = plane_cols(g.N, g.strips);
  const int rows0 = g.K / Frag<BITS>::EPS, rows1 = g.K / 32;  // word rows of the planes
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.qw, (size_t)rows0 * wcols * 4);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(NL > 0 ? g.qlo : g.qw, NL > 0 ? (size_t)rows1 * wcols * 4 : 4);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(g.zeros, (size_t)(g.K / 32 / g.upg) * g.N * 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.scales, (size_t)(g.K / 32 / g.upg) * g.N * 2);

  // A (activations) go through LDS, loaded straight into it. One load of a
  // wave fills 1 KiB: 8 rows of the 64-k slab, 128 bytes each, unpadded. The
  // 16-byte chunk c of row r sits in slot c ^ (r & 7) ^ ((r >> 3) & 1), so the
  // fragment reads of 8 (or 16) consecutive rows fall on distinct banks. Rows
  // are clamped to M - 1 (rows beyond M only feed outputs that are never
  // stored); chunks past the end of K are written as zeros instead.
  uint32_t a_voff[CQ];
  int a_c[CQ];
#pragma unroll
  for (int q = 0; q < CQ; ++q) {
    const int row = (gwave * CQ + q) * 8 + (lane >> 3);
    a_c[q] = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1);
    a_voff[q] = (uint32_t)min(m0 + row, g.M - 1) * (uint32_t)g.K * 2u + 16u * (uint32_t)a_c[q];
  }
  f16* const glds = lds + kg * NBUF * BM * BK;  // the group's activation buffers

  // B (weights) go straight to registers: each lane reads the words of its
  // fragments. With an even number of tiles per wave, tiles 2p and 2p + 1
  // take interleaved columns (column j of tile 2p + e is column 2 j + e of
  // the pair's 64), so that one 8-byte load brings a lane the words of both.
  // Columns beyond N are clamped (never stored).
  constexpr bool PAIR = TN % 2 == 0;
  constexpr int NP = PAIR ? TN / 2 : 1;
  // Weight-load instructions a wave issues per 16-k step (one per pair of
  // tiles, or per tile, and per plane): the explicit waits below count them.
  constexpr int NBI = (PAIR ? NP : TN) * (NW + NL);
  auto tile_col = [&](int t) {  // the lane's column of tile t, within the block
    return PAIR ? (BN / WN) * wn + 64 * (t >> 1) + 2 * (lane & 31) + (t & 1) : (BN / WN) * wn + 32 * t + (lane & 31);
  };
  // Per tile the lane's column (clamped to N - 1), per pair its even column
  // (clamped to N - 2): 2-byte offsets into rows of zero points and scales,
  // and byte offsets of the column's words in each plane (both columns of a
  // pair are adjacent words in either layout).
  uint32_t b_zoff[TN], p_zoff[NP];
  uint32_t b_voff[TN], p_voff[NP], b_loff[TN], p_loff[NP];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = min(n0 + tile_col(t), g.N - 1);
    b_zoff[t] = (uint32_t)n * 2u;
    b_voff[t] = plane_col(n, rows0, g.strips) * 4u;
    b_loff[t] = plane_col(n, rows1, g.strips) * 4u;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int n = min(n0 + tile_col(2 * p), g.N - 2);
    p_zoff[p] = (uint32_t)n * 2u;
    p_voff[p] = plane_col(n, rows0, g.strips) * 4u;
    p_loff[p] = plane_col(n, rows1, g.strips) * 4u;
  }

  // Slab ks into buffer buf. Slabs past the end of K (which pad the group's
  // slab count) and chunks past it are zeros: their lanes read out of range,
  // which writes zeros (a zero-length resource, or the offset x's size; x's
  // size is a multiple of 64 below 4 GiB, so that offset does not wrap).
  // Nothing here branches, so the step's instructions stay one block.
  const __amdgpu_buffer_rsrc_t rnone = make_rsrc(g.x, 0);
  const uint32_t x_bytes = (uint32_t)g.M * (uint32_t)g.K * 2u;
  // Load q of a wave's CQ loads of slab ks (each 1 KiB).
  auto dmaA_part = [&](int buf, int ks, int q) {
    const uint32_t A = lds_offset(glds + buf * BM * BK);
    const __amdgpu_buffer_rsrc_t r = (!KTAIL && ks >= nk) ? rnone : rx;
    uint32_t off = a_voff[q] + (uint32_t)ks * (BK * 2);
    if constexpr (KTAIL) off = ks * BK + 8 * a_c[q] >= g.K ? x_bytes : off;
    load_to_lds16(r, A + (gwave * CQ + q) * 1024, off);
  };
  auto dmaA = [&](int buf, int ks) {
#pragma unroll
    for (int q = 0; q < CQ; ++q) dmaA_part(buf, ks, q);
  };
  // Rows of the lane's fragments (32 apart) share their chunk swizzle.
  const int fr = (BM / WM) * wm + (lane & 31);
  const int fkey = (fr & 7) ^ ((fr >> 3) & 1);
  auto frag_a = [&](int buf, int s, int t) {
    const f16* A = glds + buf * BM * BK;
    return *reinterpret_cast<const f16x8*>(A + (fr + 32 * t) * BK + 8 * ((2 * s + kc) ^ fkey));
  };

  // Weight words of one k-step for all TN tiles, plus the step's zero point
  // and scale (the pre-scaled path) per tile.
  struct BStep {
    uint32_t w[TN][NW];
    uint32_t l[TN][NL > 0 ? NL : 1];
  };
  auto loadB = [&](BStep& S, int ks_in, int s) {
    const int ks = min(ks_in, nk - 1);
    const bool past = KTAIL && ks * BK + 16 * s >= g.K;  // this step is past the end of K: read row 0
    // kc is a lane property: it goes in the per-lane offset
    const uint32_t kcoff = past ? 0u : (BITS == 8 ? 2u * kc : (BITS == 4 ? (uint32_t)kc : 0u)) * (uint32_t)wrs * 4u;
    if constexpr (PAIR) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int row0 = past ? 0 : frag_row<BITS>(ks, s, 0, w);
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, p_voff[p] + kcoff, (uint32_t)row0 * (uint32_t)wrs * 4u, kWeightPolicy);
          S.w[2 * p][w] = v.x;
          S.w[2 * p + 1][w] = v.y;
        }
        if constexpr (NL > 0) {
          const int lrow = past ? 0 : ks * 2 + (s >> 1);
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rl, p_loff[p], (uint32_t)lrow * (uint32_t)wrs * 4u, kWeightPolicy);
          S.l[2 * p][0] = v.x;
          S.l[2 * p + 1][0] = v.y;
        }
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int row0 = past ? 0 : frag_row<BITS>(ks, s, 0, w);
        S.w[t][w] = __builtin_amdgcn_raw_buffer_load_b32(rw, b_voff[t] + kcoff, (uint32_t)row0 * (uint32_t)wrs * 4u, kWeightPolicy);
      }
      if constexpr (NL > 0) {
        const int lrow = past ? 0 : ks * 2 + (s >> 1);
        S.l[t][0] = __builtin_amdgcn_raw_buffer_load_b32(rl, b_loff[t], (uint32_t)lrow * (uint32_t)wrs * 4u, kWeightPolicy);
      }
    }
  };
  // Zero points and scales of this lane's TN columns: once (one group per
  // column) or per slab. With paired tiles the lane's two columns are
  // adjacent, and one 4-byte load brings both (tile 2p in the low half).
  constexpr int NZ = PAIR ? NP : TN;
  struct ZS {
    uint32_t z[NZ][NG], s[NZ][NG];
  };
  auto loadZS = [&](ZS& Z, int ks_in) {
    const int ks = min(ks_in, nk - 1);
#pragma unroll
    for (int h = 0; h < NG; ++h) {
      const int u = POST_SCALE ? 0 : min(ks * 2 + h, g.K / 32 - 1);
      const int grp = POST_SCALE ? 0 : (g.upg_log2 >= 0 ? (u >> g.upg_log2) : u / g.upg);
#pragma unroll
      for (int q = 0; q < NZ; ++q) {
        if constexpr (PAIR) {
          Z.z[q][h] = __builtin_amdgcn_raw_buffer_load_b32(rz, p_zoff[q], (uint32_t)grp * (uint32_t)g.N * 2u, 0);
          Z.s[q][h] = __builtin_amdgcn_raw_buffer_load_b32(rs, p_zoff[q], (uint32_t)grp * (uint32_t)g.N * 2u, 0);
        } else {
          Z.z[q][h] = __builtin_amdgcn_raw_buffer_load_b16(rz, b_zoff[q], (uint32_t)grp * (uint32_t)g.N * 2u, 0);
          Z.s[q][h] = __builtin_amdgcn_raw_buffer_load_b16(rs, b_zoff[q], (uint32_t)grp * (uint32_t)g.N * 2u, 0);
        }
      }
    }
  };
  // Bits of tile t's zero point / scale for 16-k step s.
  auto zbits = [&](const ZS& Z, int t, int s) -> uint16_t {
    const int h = NG == 2 ? (s >> 1) : 0;
    return PAIR ? (uint16_t)(Z.z[t >> 1][h] >> (16 * (t & 1))) : (uint16_t)Z.z[t][h];
  };
  auto sbits = [&](const ZS& Z, int t, int s) -> uint16_t {
    const int h = NG == 2 ? (s >> 1) : 0;
    return PAIR ? (uint16_t)(Z.s[t >> 1][h] >> (16 * (t & 1))) : (uint16_t)Z.s[t][h];
  };
  // One group per column: c = -(1024 + z) rounded to fp16, per column. For
  // |z| < 1024 it is an integer, and 1024 + q + c = q - round(z) exactly, so
  // codes dequantize with one packed add. The remainder z - round(z) (zero
  // for integer zero points) is taken out in the epilogue.
  f16x2 zc[TN];
  float czf[TN];  // bf16 data, one group per column: 1024 + z in fp32
  // Steps past the end of K (and the padding slab) need no masking here:
  // their activations are stored as zeros, and the weights they meet are
  // finite values of row 0 or of the last slab.
  auto frag_b = [&](auto fast_tag, const BStep& S, const ZS& Z, int t, int s) {
    constexpr bool FAST = decltype(fast_tag)::value;
    uint32_t h[4], d[4];
    frag_codes<BITS>(S.w[t], S.l[t], kc, s, h);
    if constexpr (BF) {
      // (1024 + q) - (1024 + z) in fp32 (times the group's scale), one rounding to bf16
      float cz, sc = 1.f;
      if constexpr (POST_SCALE) {
        cz = czf[t];
      } else {
        cz = 1024.f + bits_to_float<true>(zbits(Z, t, s));
        sc = bits_to_float<true>(sbits(Z, t, s));
      }
      // fma(h, 1, -cz) is h - cz with one rounding; with the 1 kept opaque
      // the compiler converts the fp16 half inside the mixed-precision FMA
      // (v_fma_mix_f32) instead of a conversion and a subtraction.
      float one = 1.f;
      asm("" : "+v"(one));
      // With a group scale, (h - cz) * s is one FMA h * s - cz * s (the
      // product cz * s rounded to fp32, far inside the bf16 result's rounding).
      const float f = POST_SCALE ? one : sc, c = POST_SCALE ? -cz : -cz * sc;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const f16x2 hp = as_f16x2(h[p]);
        d[p] = pack_bf16(__builtin_fmaf((float)hp.x, f, c), __builtin_fmaf((float)hp.y, f, c));
      }
    } else if constexpr (FAST) {
#pragma unroll
      for (int p = 0; p < 4; ++p) d[p] = as_u32(as_f16x2(h[p]) + zc[t]);
    } else if constexpr (BITS == 4 && !POST_SCALE) {
      // A byte of two codes in both halves of 1024.0, masked to the even
      // code at mantissa bit 0 and the odd one at bit 4 (1024 + q0 and
      // 1024 + 16 q1); one packed FMA by (1, 1/16) less (1024, 64) gives the
      // codes exactly. Then (q - z) * s as below, the same roundings.
      const f16x2 ee = f16x2{(f16)1.f, (f16)0.0625f};
      const f16x2 mm = f16x2{(f16)(-1024.f), (f16)(-64.f)};
      const f16 zh = __builtin_bit_cast(f16, zbits(Z, t, s));
      const f16 sh = __builtin_bit_cast(f16, sbits(Z, t, s));
      const f16x2 zz = f16x2{(f16)-zh, (f16)-zh};
      const f16x2 ss = f16x2{sh, sh};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t hp = __builtin_amdgcn_perm(0x64646464u, S.w[t][0], 0x04000400u | (uint32_t)p | ((uint32_t)p << 16)) & 0x64F0640Fu;
        d[p] = as_u32((__builtin_elementwise_fma(as_f16x2(hp), ee, mm) + zz) * ss);
      }
    } else {
      const f16x2 m1024 = f16x2{(f16)(-1024.f), (f16)(-1024.f)};
      const f16 zh = __builtin_bit_cast(f16, zbits(Z, t, s));
      const f16x2 zz = f16x2{(f16)-zh, (f16)-zh};
      if constexpr (POST_SCALE) {
#pragma unroll
        for (int p = 0; p < 4; ++p) d[p] = as_u32((as_f16x2(h[p]) + m1024) + zz);
      } else {
        const f16 sh = __builtin_bit_cast(f16, sbits(Z, t, s));
        const f16x2 ss = f16x2{sh, sh};
#pragma unroll
        for (int p = 0; p < 4; ++p) d[p] = as_u32(((as_f16x2(h[p]) + m1024) + zz) * ss);
      }
    }
    return __builtin_bit_cast(f16x8, u32x4{d[0], d[1], d[2], d[3]});
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Register sets: weight words and zero/scale values of two slabs in flight,
  // and the A and B fragments of the current and next 16-k step (set s % 2).
  // Indices are compile-time constants throughout, so nothing is copied
  // between sets.
  BStep B0[4], B1[4];
  ZS Z0, Z1;
  f16x8 fa[2][TM];
  f16x8 fb[2][TN];

  // One 64-k slab: four 16-k steps of TM x TN MFMAs. While a step's MFMAs
  // run, the next step's A fragments are read from LDS and its weight words
  // dequantized; the registers those words held are refilled right away
  // with the same step two slabs on. Activation slabs rotate through three
  // LDS buffers: slab i + 1, requested during step 3 of the slab before, is
  // stored during step 2 into a buffer last read two slabs ago, and the one
  // barrier per slab sits before step 3, whose next-step reads are the first
  // of slab i + 1.
  auto slab = [&](auto fast_tag, int i, BStep (&Bc)[4], BStep (&Bn)[4], ZS& Zc, ZS& Zn) __attribute__((always_inline)) {
    const int cur = i % NBUF, nxt = (i + 1) % NBUF;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // Scheduling fence: each step's instructions stay in their step.
      __builtin_amdgcn_sched_barrier(0);
      if (s == 3) {
        // This wave's loads of slab i + 1 are done: loads complete in order,
        // and at least this many were issued after its last one. Whole
        // slabs (issued NBUF - 1 slabs ago): the weight loads of
        // 4 (NBUF - 2) + 3 steps. Spread slabs (last quarter issued in step 2
        // of slab i + 2 - NBUF): the weight loads and one quarter of each of
        // 4 (NBUF - 2) steps.
        QMM_WAIT_VMCNT(cmin(SPREAD ? 4 * (NBUF - 2) * (NBI + 1) : (4 * (NBUF - 2) + 3) * NBI, 63));
        __syncthreads();  // slab i + 1 is in LDS
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          if constexpr (BF)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[s & 1][a]),
                                                                 __builtin_bit_cast(bf16x8, fb[s & 1][b]), acc[a][b], 0, 0, 0);
          else
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[s & 1][a], fb[s & 1][b], acc[a][b], 0, 0, 0);
        }
#pragma unroll
      for (int t = 0; t < TM; ++t) fa[(s + 1) & 1][t] = s < 3 ? frag_a(cur, s + 1, t) : frag_a(nxt, 0, t);
      if (s < 3) {
#pragma unroll
        for (int t = 0; t < TN; ++t) fb[(s + 1) & 1][t] = frag_b(fast_tag, Bc[s + 1], Zc, t, s + 1);
        loadB(Bc[s + 1], gslab(i + 2), s + 1);
      } else {
#pragma unroll
        for (int t = 0; t < TN; ++t) fb[0][t] = frag_b(fast_tag, Bn[0], Zn, t, 0);
        loadB(Bn[0], gslab(i + 3), 0);
      }
      if (!POST_SCALE && s == 3) loadZS(Zc, gslab(i + 2));
      if constexpr (SPREAD) {
        // A slab's four loads go out one per step: the first into slab i's
        // buffer right after the barrier that ends its reads, the other three
        // in steps 0-2 of the next slab (slab i + 2 into the buffer of slab
        // i - 1, whose reads ended before the last barrier).
        if (s == 3) dmaA_part(cur, gslab(i + NBUF), 0);
        else dmaA_part((i + NBUF - 1) % NBUF, gslab(i + NBUF - 1), s + 1);
      } else {
        if (s == 3) dmaA(cur, gslab(i + NBUF));  // every wave is past its reads of slab i
      }
      // Interleave: each MFMA is followed by a share of the step's other work.
      constexpr int NM = TM * TN;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // an LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // vector ALU
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // a global load
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Slabs run in pairs; an odd count is padded with a slab whose activations
  // and weights are zero (it adds nothing), so that the loop keeps one shape
  // and the accumulators one place.
  auto run = [&](auto fast_tag) __attribute__((always_inline)) {
    for (int i = 0; i < ni; i += 2) {
      slab(fast_tag, i, B0, B1, Z0, POST_SCALE ? Z0 : Z1);
      slab(fast_tag, i + 1, B1, B0, POST_SCALE ? Z0 : Z1, Z0);
    }
  };

#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b) dmaA(b, gslab(b));
  // the last buffer's slab: with the spread loads only its first quarter
  // here, the other three in slab 0's steps 0-2
  if constexpr (SPREAD) dmaA_part(NBUF - 1, gslab(NBUF - 1), 0);
  else dmaA(NBUF - 1, gslab(NBUF - 1));
#pragma unroll
  for (int s = 0; s < 4; ++s) loadB(B0[s], gslab(0), s);
  loadZS(Z0, gslab(0));  // with one group per column: the only zero/scale load
#pragma unroll
  for (int s = 0; s < 4; ++s) loadB(B1[s], gslab(1), s);
  if (!POST_SCALE) loadZS(Z1, gslab(1));
  QMM_WAIT_VMCNT(cmin(8 * NBI, 63));  // the first slabs' loads, issued before two slabs' weight loads
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TM; ++t) fa[0][t] = frag_a(0, 0, t);

  if constexpr (POST_SCALE) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      if constexpr (BF) {
        czf[t] = 1024.f + bits_to_float<true>(zbits(Z0, t, 0));
      } else {
        const f16 c = (f16)((f16)(-1024.f) - __builtin_bit_cast(f16, zbits(Z0, t, 0)));
        zc[t] = f16x2{c, c};
      }
    }
  }
  auto start = [&](auto fast_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TN; ++t) fb[0][t] = frag_b(fast_tag, B0[0], Z0, t, 0);
    loadB(B0[0], gslab(2), 0);
    run(fast_tag);
  };
  start(std::integral_constant<bool, POST_SCALE>{});

  // Accumulator register r of a 32 x 32 tile holds row 8 (r / 4) + 4 (lane / 32)
  // + r % 4, column lane % 32.
  auto acc_row = [&](int a, int r) { return (BM / WM) * wm + 32 * a + 8 * (r >> 2) + 4 * kc + (r & 3); };

  // One group per column: the loop subtracted c = -(1024 + z) rounded, so
  // acc = sum_k x (q - z) + delta * sum_k x with delta = z + 1024 + c (exact in
  // fp32). Blocks with a column whose delta is not zero (a zero point that is
  // not an integer) subtract delta times the row sums of x, computed here in
  // a fixed order. The barrier of the vote also ends every read of the slab
  // buffers.
  bool off = false;
  float delta[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    delta[t] = 0.f;
    if constexpr (POST_SCALE && !BF) delta[t] = (half_bits_to_float(zbits(Z0, t, 0)) + 1024.f) + (float)zc[t].x;
    off = off || delta[t] != 0.f;
  }
  QMM_WAIT_VMCNT(0);  // loads into LDS past the last slab are done before the LDS is reused
  const bool need = __syncthreads_or(off);  // every group is past its last slab
  if constexpr (KG > 1) {
    // Groups 1.. hand their sums to group 0 through LDS (over the activation
    // buffers); group 0 adds them in group order.
    float* part = reinterpret_cast<float*>(lds);
    if (kg > 0) {
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            part[(((kg - 1) * GW + gwave) * ACC + (a * TN + b) * 16 + r) * 64 + lane] = acc[a][b][r];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int j = 1; j < KG; ++j)
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              acc[a][b][r] += part[(((j - 1) * GW + gwave) * ACC + (a * TN + b) * 16 + r) * 64 + lane];
    }
  }
  if (need) {
    for (int row = tid >> 3; row < BM; row += THREADS / 8) {
      const uint16_t* xr = g.x + (size_t)min(m0 + row, g.M - 1) * g.K;
      float sum = 0.f;
      for (int k = 8 * (tid & 7); k < g.K; k += 64) {
        const f16x8 v = *reinterpret_cast<const f16x8*>(xr + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += (float)v[e];
      }
      sum += __shfl_xor(sum, 1);
      sum += __shfl_xor(sum, 2);
      sum += __shfl_xor(sum, 4);
      if ((tid & 7) == 0) rsum[row] = sum;
    }
    __syncthreads();
  }

  // Epilogue: remainder correction, scale (one group per column) and bias in
  // fp32, one rounding to fp16, stored straight from the accumulators. With
  // paired tiles a lane's two columns are adjacent: one 4-byte store, and the
  // 32 lanes of a row write 128 contiguous bytes. Tiles inside the output
  // store unconditionally; edge tiles check each row and column.
  auto emit = [&](auto need_tag, auto full_tag) __attribute__((always_inline)) {
    constexpr bool NEED = decltype(need_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int TS = PAIR ? 2 : 1;  // tiles per store
#pragma unroll
    for (int q = 0; q < TN / TS; ++q) {
      const int col = tile_col(TS * q);  // even when paired
      float sc[TS], bv[TS];
#pragma unroll
      for (int e = 0; e < TS; ++e) {
        const int n = min(n0 + col + e, g.N - 1);
        sc[e] = POST_SCALE ? bits_to_float<BF>(g.scales[n]) : 1.f;
        bv[e] = g.bias ? bits_to_float<BF>(g.bias[n]) : 0.f;
      }
      const bool col_ok = FULL || n0 + col < g.N;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row(a, r);
          uint32_t out = 0;
#pragma unroll
          for (int e = 0; e < TS; ++e) {
            float v = acc[a][TS * q + e][r];
            if constexpr (NEED) v -= delta[TS * q + e] * rsum[row];
            out |= (uint32_t)float_to_bits<BF>(v * sc[e] + bv[e]) << (16 * e);
          }
          uint16_t* dst = g.y + (size_t)(m0 + row) * g.N + n0 + col;
          if (FULL || (col_ok && m0 + row < g.M)) {
            if constexpr (PAIR) *reinterpret_cast<uint32_t*>(dst) = out;
            else *dst = (uint16_t)out;
          }
        }
    }
  };
  if (kg == 0) {  // scalar
    const bool full = m0 + BM <= g.M && n0 + BN <= g.N;
    if (need && full) emit(std::integral_constant<bool, true>{}, std::integral_constant<bool, true>{});
    else if (need) emit(std::integral_constant<bool, true>{}, std::integral_constant<bool, false>{});
    else if (full) emit(std::integral_constant<bool, false>{}, std::integral_constant<bool, true>{});
    else emit(std::integral_constant<bool, false>{}, std::integral_constant<bool, false>{});
  }
}

template <int BITS, int WM, int WN, int TM, int TN, int KG, bool BF>
hipError_t launch_tiles(GemmArgs a, hipStream_t s) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  a.mblocks = (a.M + BM - 1) / BM;
  a.nblocks = (a.N + BN - 1) / BN;
  const int nblocks = a.mblocks * a.nblocks;
  const int zm = a.upg * 32 == a.K ? 2 : (a.upg % 2 == 0 ? 1 : 0);
  const bool tail = a.K % BK != 0;
  constexpr int T = 64 * WM * WN * KG;
  if (zm == 2 && !tail) gemm_kernel<BITS, 2, false, WM, WN, TM, TN, KG, BF><<<nblocks, T, 0, s>>>(a);
  else if (zm == 2) gemm_kernel<BITS, 2, true, WM, WN, TM, TN, KG, BF><<<nblocks, T, 0, s>>>(a);
  // Groups of whole slabs make K a multiple of 64: no tail.
  else if (zm == 1) gemm_kernel<BITS, 1, false, WM, WN, TM, TN, KG, BF><<<nblocks, T, 0, s>>>(a);
  else if (!tail) gemm_kernel<BITS, 0, false, WM, WN, TM, TN, KG, BF><<<nblocks, T, 0, s>>>(a);
  else gemm_kernel<BITS, 0, true, WM, WN, TM, TN, KG, BF><<<nblocks, T, 0, s>>>(a);
  return hipGetLastError();
}

template <int BITS, bool BF>
hipError_t launch_bits(const GemmArgs& a, int tile, hipStream_t s) {
  switch (tile) {
    case 0: return launch_tiles<BITS, 2, 4, 4, 2, 1, BF>(a, s);
    case 1: return launch_tiles<BITS, 2, 2, 2, 2, 2, BF>(a, s);
    case 2: return launch_tiles<BITS, 1, 2, 2, 1, 6, BF>(a, s);
    case 3: return launch_tiles<BITS, 2, 2, 1, 1, 4, BF>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF>
hipError_t launch_dtype(const GemmArgs& a, int bits, int tile, hipStream_t s) {
  switch (bits) {
    case 1: return launch_bits<1, BF>(a, tile, s);
    case 2: return launch_bits<2, BF>(a, tile, s);
    case 3: return launch_bits<3, BF>(a, tile, s);
    case 4: return launch_bits<4, BF>(a, tile, s);
    case 8: return launch_bits<8, BF>(a, tile, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// The largest block tile whose grid still gives every CU a block: 256 x 256
// (8 waves of 128 x 64), else 128 x 128 (two K groups of 4 waves of 64 x 64),
// else 64 x 64. Smaller tiles have short slabs, so their blocks split K to
// keep more loads in flight: a 64 x 64 block's time is about its groups'
// chain of slabs (run in pairs) times the latency of one, so it takes six
// K groups of 2 waves of 64 x 32 where that chain is shorter than with four
// groups of 4 waves of 32 x 32 (K of 2048 and more), else the four groups.
GemmPlan gemm_plan(int M, int K, int N, DeviceTopo topo) {
  static const int kShapes[4][3] = {{256, 256, 1}, {128, 128, 2}, {64, 64, 6}, {64, 64, 4}};
  const int cus = topo.cus > 0 ? topo.cus : 256;
  auto blocks = [&](int bm, int bn) { return (((long long)M + bm - 1) / bm) * (((long long)N + bn - 1) / bn); };
  int tile = 3;
  if (blocks(256, 256) >= cus) {
    tile = 0;
  } else if (blocks(128, 128) >= cus) {
    tile = 1;
  } else {
    const int nk = (int)(((long long)K + BK - 1) / BK);
    auto chain = [&](int kg) {
      const int n = (nk + kg - 1) / kg;
      return n + (n & 1);
    };
    if (chain(6) < chain(4)) tile = 2;
  }
  GemmPlan p;
  p.tile = tile;
  p.bm = kShapes[tile][0];
  p.bn = kShapes[tile][1];
  p.kgroups = kShapes[tile][2];
  p.waves = tile == 0 ? 8 : (tile == 1 ? 8 : (tile == 2 ? 12 : 16));
  p.blocks = blocks(p.bm, p.bn);
  p.xcds = topo.xcds > 0 ? topo.xcds : 8;
  p.cus = cus;
  return p;
}

hipError_t launch_gemm(const uint16_t* x, int M, int K, const uint32_t* qw, const uint32_t* qlo,
                       const uint16_t* zeros, const uint16_t* scales, const uint16_t* bias, int N, int bits,
                       int group_size, uint16_t* y, bool bf16, bool strips, DeviceTopo topo, hipStream_t s) {
  GemmArgs a;
  a.strips = strips ? 1 : 0;
  a.xcds = topo.xcds > 0 ? topo.xcds : 8;
  a.cus = topo.cus > 0 ? topo.cus : 256;
  a.x = x;
  a.qw = qw;
  a.qlo = qlo;
  a.zeros = zeros;
  a.scales = scales;
  a.bias = bias;
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.upg = group_rows(K, group_size) / 32;
  a.upg_log2 = -1;
  for (int l = 0; l < 31; ++l)
    if ((1 << l) == a.upg) a.upg_log2 = l;
  const int tile = gemm_plan(M, K, N, topo).tile;
  return bf16 ? launch_dtype<true>(a, bits, tile, s) : launch_dtype<false>(a, bits, tile, s);
}

}  // namespace qmm
