// Prefill product y = x @ dequant(W) for any M on gfx950's matrix cores.
//
// What is computed is the dense product of x with the dequantized weight
// (dashq_kernel.py, TritonQuantLinear.forward batched path and
// dequantize_weight; GPTQModel-Compatible Triton Kernel README, overview: the
// dequantization is fused into the product instead of materialising W).
//
// Design:
//  * Block tile 256 x 256, K in slabs of 64; 4 waves in a 2 x 2 arrangement,
//    each wave a 128 x 128 sub-tile of 8 x 8 V_MFMA_F32_16X16X32_F16
//    accumulators (256 fp32 accumulation registers per lane).
//  * Both operands are staged in LDS as fp16 with k contiguous: A[m][k] and
//    B[n][k], row pitch 72 halves, so the 16-byte fragment reads of 8 lanes
//    touch 32 distinct banks. Two LDS buffers alternate between slabs.
//  * Global loads run two slabs ahead into two register sets, so a slab's
//    latency is covered by two slabs of matrix-core work.
//  * Packed words are dequantized once per block on their way into LDS: each
//    thread owns one column of the slab (64 codes), turns codes into halves
//    with the 1024.0 mantissa trick (byte permute for 8-bit) and subtracts
//    1024, then the zero point (exact for integer zero points). With one
//    group per column
//    (group_size -1) the scale is applied to the fp32 accumulator in the
//    epilogue; otherwise each half is multiplied by its group's scale before
//    it is stored (one fp16 rounding).
//  * Each 64-k slab is two 32-k sub-steps. A fragments are read from LDS one
//    step ahead of their MFMAs; during the second sub-step the next slab is
//    dequantized into the other LDS buffer and the weights of the slab after
//    it are requested from memory. The activation loads of the next slab are
//    pinned to the start of the slab so their latency is covered.
//  * The epilogue stages the fp16 tile through LDS and writes rows with
//    16-byte stores.
//  * Block ids are remapped so that each of the 8 XCDs (own L2 each) works on
//    a contiguous run of tiles that share weight and activation panels.
#include "common.h"

namespace qmm {
namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int LDK = BK + 8;  // halves per LDS row of a staged slab
constexpr int LDY = BN + 8;  // halves per LDS row of the staged output tile
constexpr int kLdsHalves = 2 * (BM + BN) * LDK;  // two slab buffers; the output tile reuses them
static_assert(BM * LDY <= kLdsHalves, "output tile must fit in the slab buffers");

struct GemmArgs {
  const uint16_t* x;
  const uint32_t* qw;
  const uint32_t* qlo;
  const uint16_t* zeros;
  const uint16_t* scales;
  uint16_t* y;
  int M, K, N;
  int upg;       // 32-row units per group
  int upg_log2;  // log2(upg) if a power of two, else -1
  int mblocks, nblocks;
};

// Word rows of one plane a 64-k slab spans.
template <int BITS> struct Slab;
template <> struct Slab<8> { static constexpr int R = 16, RLO = 0, EPS = 4; };
template <> struct Slab<4> { static constexpr int R = 8, RLO = 0, EPS = 8; };
template <> struct Slab<2> { static constexpr int R = 4, RLO = 0, EPS = 16; };
template <> struct Slab<3> { static constexpr int R = 4, RLO = 2, EPS = 16; };

// One slab's weight words held by one thread (its column), plus the zero
// point and scale of each 32-k half when every group has its own.
template <int BITS, bool POST_SCALE> struct StageB {
  uint32_t w[Slab<BITS>::R];
  uint32_t l[Slab<BITS>::RLO > 0 ? Slab<BITS>::RLO : 1];
  uint16_t z[POST_SCALE ? 1 : 2], s[POST_SCALE ? 1 : 2];
};

// Four fp16 pairs 1024 + q for codes k = 8c .. 8c + 7 of a 64-k slab, k
// ascending (pair i = codes 8c + 2i, 8c + 2i + 1), from the words of one
// column covering the slab.
template <int BITS>
__device__ __forceinline__ void codes8(const uint32_t* w, const uint32_t* wl, int c, uint32_t (&h)[4]) {
  if constexpr (BITS == 8) {
    // byte permute: (byte, 0x64, byte, 0x64) = halves 1024 + q
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      h[2 * r] = __builtin_amdgcn_perm(0x64646464u, w[2 * c + r], 0x04010400u);
      h[2 * r + 1] = __builtin_amdgcn_perm(0x64646464u, w[2 * c + r], 0x04030402u);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t t = w[c] >> (8 * p);
      h[p] = (t & 0xFu) | ((t << 12) & 0xF0000u) | kMagic1024x2;
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t t = w[c >> 1] >> (16 * (c & 1) + 4 * p);
      h[p] = (t & 0x3u) | ((t << 14) & 0x30000u) | kMagic1024x2;
    }
  } else {
    const uint32_t hw = w[c >> 1] >> (16 * (c & 1));
    const uint32_t lw = wl[c >> 2] >> (8 * (c & 3));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = (((hw >> (4 * p)) & 0x3u) << 1) | ((lw >> (2 * p)) & 1u);
      const uint32_t b = (((hw >> (4 * p + 2)) & 0x3u) << 1) | ((lw >> (2 * p + 1)) & 1u);
      h[p] = a | (b << 16) | kMagic1024x2;
    }
  }
}

__device__ __forceinline__ int remap_block(int pid, int nblocks) {
  // Dispatch places block ids round-robin on the 8 XCDs; give each XCD a
  // contiguous range of tile ids so neighbouring tiles share its L2.
  if (nblocks % 8 != 0) return pid;
  return (pid % 8) * (nblocks / 8) + pid / 8;
}

// A raw buffer resource over `bytes` bytes at p (out-of-range reads return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
constexpr int kNonTemporal = 2;  // buffer-load cache policy: streamed data

// Scheduling-group mask of vector-memory reads (AMDGPU sched_group_barrier).
constexpr int kSchedVmemRead = 0x020;

template <int BITS, bool POST_SCALE, bool KTAIL>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) f16 lds[kLdsHalves];
  constexpr int R = Slab<BITS>::R;
  constexpr int RLO = Slab<BITS>::RLO;
  constexpr int EPS = Slab<BITS>::EPS;
  using SB = StageB<BITS, POST_SCALE>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int i16 = lane & 15, j4 = lane >> 4;

  const int tile = remap_block(blockIdx.x, g.mblocks * g.nblocks);
  const int nb = tile / g.mblocks;
  const int mb = tile - nb * g.mblocks;
  const int m0 = mb * BM, n0 = nb * BN;
  const int nk = (g.K + BK - 1) / BK;

  // Buffer resources: every global load below is a 32-bit per-lane offset
  // plus a scalar per-slab offset, which keeps address arithmetic out of the
  // vector registers.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.x, (size_t)g.M * g.K * 2);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.qw, (size_t)(g.K / EPS) * g.N * 4);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(RLO > 0 ? g.qlo : g.qw, RLO > 0 ? (size_t)(g.K / 32) * g.N * 4 : 4);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(g.zeros, (size_t)(g.K / 32 / g.upg) * g.N * 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.scales, (size_t)(g.K / 32 / g.upg) * g.N * 2);

  // A loader: rows a_row + 32 i (clamped to M - 1: rows beyond M only feed
  // outputs that are never stored), 8 halves at column chunk a_chk.
  const int a_row = tid >> 3, a_chk = tid & 7;
  uint32_t a_voff[8];  // byte offsets into x
#pragma unroll
  for (int i = 0; i < 8; ++i) a_voff[i] = (uint32_t)(min(m0 + a_row + 32 * i, g.M - 1) * g.K + 8 * a_chk) * 2u;
  // B loader: one column per thread (clamped to N - 1 likewise).
  const int b_col = min(n0 + tid, g.N - 1);
  const uint32_t b_voff = (uint32_t)b_col * 4u;

  auto loadA = [&](u32x4 (&SA)[8], int ks_in) {
    const int ks = min(ks_in, nk - 1);  // slabs past the end reload the last one (never used)
    // Chunks past the end of K (second half of the last slab when K % 64 != 0)
    // read the chunk 32 halves before instead; they are zeroed when stored.
    const uint32_t adj = (KTAIL && ks * BK + 8 * a_chk >= g.K) ? 64u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) SA[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, a_voff[i] - adj, ks * BK * 2, 0);
  };
  auto loadB = [&](SB& S, int ks_in) {
    const int ks = min(ks_in, nk - 1);
    const int row0 = ks * (BK / EPS);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // word rows past the end of K read row 0 instead (zeroed when stored)
      const int row = (!KTAIL || (row0 + r) * EPS < g.K) ? row0 + r : 0;
      S.w[r] = __builtin_amdgcn_raw_buffer_load_b32(rw, b_voff, row * g.N * 4, kNonTemporal);
    }
    if constexpr (RLO > 0) {
      const int lrow0 = ks * (BK / 32);
#pragma unroll
      for (int r = 0; r < RLO; ++r) {
        const int row = (!KTAIL || (lrow0 + r) * 32 < g.K) ? lrow0 + r : 0;
        S.l[r] = __builtin_amdgcn_raw_buffer_load_b32(rl, b_voff, row * g.N * 4, kNonTemporal);
      }
    }
    if constexpr (!POST_SCALE) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int u = min(ks * 2 + h, g.K / 32 - 1);
        const int grp = g.upg_log2 >= 0 ? (u >> g.upg_log2) : u / g.upg;
        S.z[h] = __builtin_amdgcn_raw_buffer_load_b16(rz, (uint32_t)b_col * 2u, grp * g.N * 2, 0);
        S.s[h] = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)b_col * 2u, grp * g.N * 2, 0);
      }
    }
  };

  // Zero point of this thread's column when there is one group per column.
  f16x2 zneg = f16x2{0, 0};
  if constexpr (POST_SCALE) {
    const f16 z = __builtin_bit_cast(f16, g.zeros[b_col]);
    zneg = f16x2{(f16)-z, (f16)-z};
  }

  auto storeA = [&](const u32x4 (&SA)[8], int buf, int ks) {
    f16* A = lds + buf * (BM + BN) * LDK;
    const bool tail = KTAIL && (ks * BK + 32 >= g.K);  // only the first 32-k half is inside K
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u32x4 v = SA[i];
      if (KTAIL && tail && a_chk >= 4) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(A + (a_row + 32 * i) * LDK + 8 * a_chk) = v;
    }
  };
  auto storeB = [&](const SB& S, int buf, int ks) {
    f16* B = lds + buf * (BM + BN) * LDK + BM * LDK;
    const bool tail = KTAIL && (ks * BK + 32 >= g.K);
    const f16x2 m1024 = f16x2{(f16)(-1024.f), (f16)(-1024.f)};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t h[4], d[4];
      codes8<BITS>(S.w, S.l, c, h);
      if constexpr (POST_SCALE) {
#pragma unroll
        for (int p = 0; p < 4; ++p) d[p] = as_u32((as_f16x2(h[p]) + m1024) + zneg);
      } else {
        const f16 zh = __builtin_bit_cast(f16, S.z[c >> 2]);
        const f16 sh = __builtin_bit_cast(f16, S.s[c >> 2]);
        const f16x2 zz = f16x2{(f16)-zh, (f16)-zh}, ss = f16x2{sh, sh};
#pragma unroll
        for (int p = 0; p < 4; ++p) d[p] = as_u32(((as_f16x2(h[p]) + m1024) + zz) * ss);
      }
      u32x4 v = u32x4{d[0], d[1], d[2], d[3]};
      if (KTAIL && tail && c >= 4) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(B + tid * LDK + 8 * c) = v;
    }
  };

  auto frag_a = [&](int buf, int s, int t) {
    const f16* A = lds + buf * (BM + BN) * LDK;
    return *reinterpret_cast<const f16x8*>(A + (128 * wm + 16 * t + i16) * LDK + 32 * s + 8 * j4);
  };
  auto frag_b = [&](int buf, int s, int t) {
    const f16* B = lds + buf * (BM + BN) * LDK + BM * LDK;
    return *reinterpret_cast<const f16x8*>(B + (128 * wn + 16 * t + i16) * LDK + 32 * s + 8 * j4);
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 SA[8];
  SB Pn1, Pn2;  // weight words of the next slab and of the one after it
  f16x8 bf[8], af;

  loadA(SA, 0);
  loadB(Pn1, 0);
  loadB(Pn2, 1);
  storeA(SA, 0, 0);
  storeB(Pn1, 0, 0);
  Pn1 = Pn2;
  loadB(Pn2, 2);
  __syncthreads();
  af = frag_a(0, 0, 0);
#pragma unroll
  for (int b = 0; b < 8; ++b) bf[b] = frag_b(0, 0, b);

  // One slab per iteration: two sub-steps of 64 MFMAs each.
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    loadA(SA, ks + 1);
    // sub-step 0; A fragments are read one ahead of their MFMAs
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const f16x8 a_now = af;
      af = frag_a(cur, t < 7 ? 0 : 1, t < 7 ? t + 1 : 0);
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[t][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_now, bf[b], acc[t][b], 0, 0, 0);
    }
    // the activation loads of the next slab go out first
    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 8, 0);
#pragma unroll
    for (int b = 0; b < 8; ++b) bf[b] = frag_b(cur, 1, b);
    // sub-step 1, staging the next slab in the other buffer under it and
    // requesting the weight words of the slab after the next
    storeB(Pn1, cur ^ 1, ks + 1);
    Pn1 = Pn2;
    loadB(Pn2, ks + 3);
    storeA(SA, cur ^ 1, ks + 1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const f16x8 a_now = af;
      if (t < 7) af = frag_a(cur, 1, t + 1);
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[t][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_now, bf[b], acc[t][b], 0, 0, 0);
    }
    __syncthreads();
    af = frag_a(cur ^ 1, 0, 0);
#pragma unroll
    for (int b = 0; b < 8; ++b) bf[b] = frag_b(cur ^ 1, 0, b);
  }

  // Epilogue: scale (one group per column), round to fp16, stage the tile in
  // LDS, then write rows with 16-byte stores.
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int col = 128 * wn + 16 * b + i16;
    float s = 1.f;
    if constexpr (POST_SCALE) s = half_bits_to_float(g.scales[min(n0 + col, g.N - 1)]);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) lds[(128 * wm + 16 * a + 4 * j4 + r) * LDY + col] = (f16)(acc[a][b][r] * s);
  }
  __syncthreads();
#pragma unroll 4
  for (int c = tid; c < BM * (BN / 8); c += kThreads) {
    const int row = c / (BN / 8), chunk = c - row * (BN / 8);
    const int gr = m0 + row, gc = n0 + 8 * chunk;
    if (gr < g.M && gc < g.N)
      *reinterpret_cast<u32x4*>(g.y + (size_t)gr * g.N + gc) = *reinterpret_cast<const u32x4*>(lds + row * LDY + 8 * chunk);
  }
}

template <int BITS>
hipError_t launch_bits(const GemmArgs& a, hipStream_t s) {
  const int nblocks = a.mblocks * a.nblocks;
  const bool post = a.upg * 32 == a.K;
  const bool tail = a.K % BK != 0;
  if (post && !tail) gemm_kernel<BITS, true, false><<<nblocks, kThreads, 0, s>>>(a);
  else if (post) gemm_kernel<BITS, true, true><<<nblocks, kThreads, 0, s>>>(a);
  else if (!tail) gemm_kernel<BITS, false, false><<<nblocks, kThreads, 0, s>>>(a);
  else gemm_kernel<BITS, false, true><<<nblocks, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, int M, int K, const uint32_t* qw, const uint32_t* qlo,
                       const uint16_t* zeros, const uint16_t* scales, int N, int bits, int group_size,
                       uint16_t* y, hipStream_t s) {
  GemmArgs a;
  a.x = x;
  a.qw = qw;
  a.qlo = qlo;
  a.zeros = zeros;
  a.scales = scales;
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.upg = group_rows(K, group_size) / 32;
  a.upg_log2 = -1;
  for (int l = 0; l < 31; ++l)
    if ((1 << l) == a.upg) a.upg_log2 = l;
  a.mblocks = (M + BM - 1) / BM;
  a.nblocks = (N + BN - 1) / BN;
  switch (bits) {
    case 2: return launch_bits<2>(a, s);
    case 3: return launch_bits<3>(a, s);
    case 4: return launch_bits<4>(a, s);
    case 8: return launch_bits<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmm
