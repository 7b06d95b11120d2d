// The wave-local decode product (see the description below), instantiated
// per code width by gemv_wave_b<bits>.hip.
#pragma once

#include "gemv_common.h"

namespace qmm {
namespace {

// ---- wave-local decode product ---------------------------------------------
// The plan takes this kernel when one block per column strip covers all of K
// (no split along K), every wave gets the same number UPW of 32-row units
// (a compile-time constant, so the unit loop is unrolled and carries no
// scalar bookkeeping per unit), groups hold a power-of-two number of units
// (or one group spans K) and the block's activations fit its staging area:
//
//  * Every wave requests, in this order: activation slots, the raw scales
//    and zero points of the groups its units touch (into registers), and
//    the weight words of all its units.
//  * The activations are written to LDS in the operand order of the matrix
//    cores (once per wave or block, where the lanes of a lane group would
//    otherwise each permute the same 16 bytes). Each wave stages the slots
//    of its own units in an area of its own and waits for those only,
//    except for one row at 16 units per wave, where the block stages them
//    and meets at one barrier. Activations come from L2, but a later wave's
//    requests queue behind the earlier waves' weight words, so a block-wide
//    barrier can wait long for the last wave's (4 us against 1.3 us for the
//    first wave's at M = 8).
//  * Each wave then runs its units as their words arrive (loads complete in
//    order). The wave's units form GPW (1, 2 or 4) groups of equal size, a
//    compile-time structure: no scalar bookkeeping per unit.
//  * fp16 data: the codes become fp16 subnormals with bit operations only
//    (no zero point, no offset), the matrix cores form sum x q and sum x per
//    group, and s (q - z) is applied to those two fp32 sums (any fp16 zero
//    point). The waves' fp32 results are summed through LDS in wave order
//    and rounded once.
// LDS: the staged activations (M * K / 32 * 4 slots of 16 bytes, in an area
// of 4 slots per thread, 256 per wave), later reused for the per-wave
// results (WAVES * M * 16 * VEC floats); sized at launch, at most 64 KiB.
constexpr int kWaveXPerThread = 4; // activation slots one thread stages at most

// VEC consecutive halves of a row of scales or zero points, as loaded: a
// single half stays a 16-bit value (widening it right after the load would be
// an instruction that waits for the load), two or four halves are 32-bit words.
template <int VEC> struct HalfWords {
  static constexpr int N = VEC == 4 ? 2 : 1;
  typedef typename std::conditional<VEC == 1, uint16_t, uint32_t>::type T;
};
template <int VEC>
__device__ __forceinline__ void load_halves(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                            typename HalfWords<VEC>::T (&h)[HalfWords<VEC>::N]) {
  if constexpr (VEC == 1) {
    h[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else if constexpr (VEC == 2) {
    h[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else {
    const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    h[0] = t.x;
    h[1] = t.y;
  }
}
template <int VEC>
__device__ __forceinline__ uint16_t half_bits(const typename HalfWords<VEC>::T (&h)[HalfWords<VEC>::N], int v) {
  if constexpr (VEC == 1) return h[0];
  else return (uint16_t)(h[v >> 1] >> (16 * (v & 1)));
}

// fp16 data: the codes enter the matrix cores as fp16 subnormals 2^e q 2^-24
// (decode8 with SUB; e = code_exp_sub, the code's place in the mantissa), which
// the matrix cores take exactly. The activations are staged with element
// (p, hi) scaled by 2^-e, so every product is x q 2^-24 whatever the place,
// and a B operand of 2^e gives the sum of x over the same k. Per group, the
// dequantization s (q - z) is then applied to the two sums:
// s 2^24 (sum x q 2^-24 - z 2^-24 sum x), any fp16 zero point, no offset.
template <int BITS>
__device__ __forceinline__ u32x4 x_prescaled(u32x4 a) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (code_exp_sub<BITS>(p, 0) != 0 || code_exp_sub<BITS>(p, 1) != 0)
      a[p] = as_u32(as_f16x2(a[p]) * f16x2{(f16)(1.0f / (float)(1 << code_exp_sub<BITS>(p, 0))),
                                           (f16)(1.0f / (float)(1 << code_exp_sub<BITS>(p, 1)))});
  }
  return a;
}
template <int BITS>
__device__ __forceinline__ f16x8 place_ones() {
  f16x8 o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    o[2 * p] = (f16)(float)(1 << code_exp_sub<BITS>(p, 0));
    o[2 * p + 1] = (f16)(float)(1 << code_exp_sub<BITS>(p, 1));
  }
  return o;
}

template <int BITS, int VEC, int WAVES, int UPW, int GPW, bool BF, bool M1>
__global__ __launch_bounds__(64 * WAVES) void gemv_wave_kernel(GemvArgs g) {
  constexpr int NW = Bits<BITS>::NW;
  constexpr int NPC = kPairClasses<BITS>;
  constexpr int COLS = 16 * VEC;
  constexpr int THREADS = 64 * WAVES;
  constexpr int HW = HalfWords<VEC>::N;
  constexpr int GU = UPW / GPW;        // units per group within the wave
  constexpr int U = WAVES * UPW;       // K / 32
  constexpr bool SPLIT_E = BITS == 1;
  typedef typename HalfWords<VEC>::T HT;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane >> 4;
  const int cl = lane & 15;
  // A grid of few strips runs on XCD 0 alone: workgroups are dealt to the
  // XCDs round-robin by linear id, and XCD 0 starts its blocks first (the
  // others up to ~0.7 us later on MI355X). The blocks dealt to the other XCDs
  // return before touching memory.
  if (g.one_xcd > 1 && blockIdx.x % g.one_xcd != 0) return;
  const int strip = g.one_xcd > 1 ? (int)blockIdx.x / g.one_xcd : xcd_strip(blockIdx.x, gridDim.x, g.xcd_log2);
  const int n0 = strip * COLS;
  const int nc = n0 + VEC * cl;
  const int ncc = nc < g.N ? nc : 0;
  const int m = M1 ? 0 : (cl < g.M ? cl : 0);
  const int ua = wave * UPW;
  // First group of the wave and the number of groups: GPW groups of GU units
  // each, or (GPW == 1) the one group holding all of the wave's units.
  const int g0 = GPW > 1 ? wave * GPW : (ua >> g.gl);
  const int G = GPW > 1 ? WAVES * GPW : (U >> g.gl > 0 ? U >> g.gl : 1);
  u32x4* xs = reinterpret_cast<u32x4*>(dyn_lds);
  float* red = reinterpret_cast<float*>(dyn_lds);  // reused after the units

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.x, (size_t)g.M * g.K * 2);
  const long long wcols = plane_cols(g.N, g.strips);
  const int wrs = plane_row_stride(g.N, g.strips);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.qw, (size_t)U * unit_rows<BITS>(0) * wcols * 4);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(BITS == 3 ? g.qlo : g.qw, (size_t)U * unit_rows<BITS>(NW - 1) * wcols * 4);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.scales, (size_t)G * g.N * 2);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(g.zeros, (size_t)G * g.N * 2);

  // ---- 1. requests, all before the first wait: activation slots, the raw
  // scales and zero points of the wave's groups, the weight words of its
  // units.
  constexpr int XROW = 4 * U;  // activation slots per row: (m, u, j) at m XROW + 4 u + j
  // One row (M1): the block stages XROW <= THREADS slots, one per thread
  // (threads past them repeat the last slot), and meets at a barrier.
  // Several rows (OWN): each wave stages its own slots (its units, every
  // row: M * UPW * 4 <= 256 of them, a limit of the plan, so at most 4 per
  // lane) in an area of its own and waits for nothing else: a wave whose
  // activations arrive early starts its units while the other waves' still
  // come in (later waves' requests queue behind the earlier waves' weight
  // words).
  // One row with fewer than 16 units per wave: the block-wide staging would
  // leave the activation requests to the first waves only (one slot per
  // thread), so the waves stage their own there too (measured faster; with
  // 16 units per wave each wave's threads already hold its own slots, and
  // the block's barrier measured faster than none).
  constexpr bool OWN = QMM_GEMV_WAVE_X && (!M1 || UPW < 16);
  constexpr int WSLOTS = 64 * kWaveXPerThread;  // slots of a wave's own area
  constexpr int WROW = 4 * UPW;                 // a wave's slots per row: (m, c, j) at m WROW + 4 c + j
  const int xslots = OWN ? g.M * WROW : (M1 ? XROW : g.M * XROW);
  const int xpt = OWN ? (xslots + 63) / 64 : (M1 ? 1 : (xslots + THREADS - 1) / THREADS);  // wave-uniform
  const int xbase = OWN ? wave * WSLOTS : 0;  // first slot of the thread's writes
  u32x4 xraw[kWaveXPerThread];
#pragma unroll
  for (int i = 0; i < kWaveXPerThread; ++i) {
    if (i < xpt) {  // scalar (compile-time for one row)
      if constexpr (OWN) {
        const int sl = min(lane + 64 * i, xslots - 1);
        const int mm = sl / WROW, rem = sl % WROW;
        xraw[i] = load_x_slot<BITS>(rx, (uint32_t)(mm * g.K + 32 * (ua + (rem >> 2)) + x_first<BITS>(rem & 3)) * 2u);
      } else {
        const int sl = min(tid + THREADS * i, xslots - 1);
        const int mm = M1 ? 0 : sl / XROW, rem = M1 ? sl : sl % XROW;
        xraw[i] = load_x_slot<BITS>(rx, (uint32_t)(mm * g.K + 32 * (rem >> 2) + x_first<BITS>(rem & 3)) * 2u);
      }
    }
  }
  // Scales and zero points of the wave's groups. With several rows and
  // several groups, lane group j requests those of group slot j % GPW only
  // and the lanes exchange them after the staging (a cross-lane permute per
  // value): two small requests per lane instead of 2 GPW, each a separate
  // trip to memory (measured faster there, slower for one row). The zero
  // points a lane requests for itself are the ones it checks for the exact
  // one-operation dequantization (VEC values per lane instead of GPW * VEC).
  constexpr bool SHARE = QMM_GEMV_SZ_SHARE && GPW > 1 && !M1;
  HT sraw[GPW][HW], zraw[GPW][HW];
  HT sown[HW], zchk[HW];
  if constexpr (SHARE) {
    const uint32_t off = ((uint32_t)(g0 + (j & (GPW - 1))) * (uint32_t)g.N + (uint32_t)ncc) * 2u;
    load_halves<VEC>(rs, off, sown);
    load_halves<VEC>(rz, off, zchk);
  } else {
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const uint32_t off = ((uint32_t)(g0 + gi) * (uint32_t)g.N + (uint32_t)ncc) * 2u;
      load_halves<VEC>(rs, off, sraw[gi]);
      load_halves<VEC>(rz, off, zraw[gi]);
    }
  }
  uint32_t woff[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w)
    woff[w] = (plane_col(ncc, U * unit_rows<BITS>(w), g.strips) + (uint32_t)(lane_row<BITS>(j, w) * wrs)) * 4u;
  typename Vec<VEC>::T wv[UPW][NW];
#pragma unroll
  for (int c = 0; c < UPW; ++c) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t soff = (uint32_t)((ua + c) * unit_rows<BITS>(w)) * (uint32_t)wrs * 4u;
      wv[c][w] = load_words<VEC>((BITS == 3 && w == 1) ? rl : rw, woff[w], soff);
    }
  }

  // ---- 2. activations into LDS in operand order; one barrier. Each thread
  // writes its xpt slots under a wave-uniform condition only (slots past the
  // activations, within the area of THREADS * kWaveXPerThread slots, receive
  // copies that are never read): a write under a per-lane condition let the
  // compiler move that slot's load after the weight requests and wait for
  // all of them before the barrier.
#pragma unroll
  for (int i = 0; i < kWaveXPerThread; ++i)
    if (i < xpt) {  // scalar condition
      const u32x4 a = x_operand<BITS>(xraw[i]);
      xs[xbase + (OWN ? lane + 64 * i : tid + THREADS * i)] = BF ? a : x_prescaled<BITS>(a);
    }
  // One row, block staging (every thread one slot, the slots of a wave's
  // units in its own lanes): the sum of x per group is the same for every
  // column, so it comes from the staged slots instead of a second
  // matrix-core product per unit. Each thread adds its slot's 8 values
  // (packed dot products with ones, fp32), into an LDS array after the slots.
  constexpr bool XSUM_LDS = QMM_GEMV_XSUM_LDS && !BF && M1 && !OWN;
  float* const ps = reinterpret_cast<float*>(xs + THREADS);
  if constexpr (XSUM_LDS) {
    const f16x2 one2 = f16x2{(f16)1.f, (f16)1.f};
    float p = __builtin_amdgcn_fdot2(as_f16x2(xraw[0].x), one2, 0.f, false);
    p = __builtin_amdgcn_fdot2(as_f16x2(xraw[0].y), one2, p, false);
    p = __builtin_amdgcn_fdot2(as_f16x2(xraw[0].z), one2, p, false);
    p = __builtin_amdgcn_fdot2(as_f16x2(xraw[0].w), one2, p, false);
    ps[tid] = p;
  }
  if constexpr (OWN) {
    // The wave reads back only what it wrote itself: LDS operations of one
    // wave take effect in order, so a compiler-level fence is enough.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  } else {
    __syncthreads();
  }
  // Nothing below (the group constants wait for the scales and zero points,
  // which come from HBM) may be scheduled above this point: the wait here
  // should be for the activations only, which come from L2.
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (SHARE) {
    // group slot gi of column cl: from lane cl of lane group gi
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int src = ((lane & 15) | (gi << 4)) << 2;
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        sraw[gi][h] = (HT)__builtin_amdgcn_ds_bpermute(src, (int)sown[h]);
        zraw[gi][h] = (HT)__builtin_amdgcn_ds_bpermute(src, (int)zchk[h]);
      }
    }
  }

  // The wave's sums of x per group: lane l holds slot 4 ua + l (the wave's
  // 64 slots); a butterfly over each group's lanes (fixed order, the same
  // result in every lane) and one lane's value per group.
  float xsg[GPW] = {};
  if constexpr (XSUM_LDS) {
    static_assert(4 * UPW == 64, "block staging gives a wave 64 slots");
    constexpr int LG = 64 / GPW;  // lanes (slots) per group within the wave
    float v = ps[4 * ua + lane];
#pragma unroll
    for (int off = 1; off < LG; off <<= 1) v += __shfl_xor(v, off);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi)
      xsg[gi] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), LG * gi));
  }

  // ---- 3. the wave's units, group by group (static).
  // fp16 data: per unit one matrix-core product of the prescaled activations
  // with the subnormal codes (sum x q 2^-24) per column set, and one with the
  // place values 2^e (sum x, shared by the VEC column sets); per group the
  // scale and zero point are applied to the two sums in fp32. bf16 data:
  // q - z is formed in fp32 per code (czf = 1024 2^-e + z, or z alone for
  // 1-bit codes) and rounded once to bf16.
  const DecodeMasks<BITS> dm = decode_masks<BITS, !BF>();
  const f16x8 ones = place_ones<BITS>();
  f32x4 total[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) total[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4* xrow = OWN ? xs + (wave * WSLOTS + m * WROW + j) : xs + (m * XROW + 4 * ua + j);  // unit ua + c at xrow[4 c]
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    float sc[VEC], czf[NPC][VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      sc[v] = bits_to_float<BF>(half_bits<VEC>(sraw[gi], v));
      if constexpr (BF) {
        const float zf = bits_to_float<BF>(half_bits<VEC>(zraw[gi], v));
#pragma unroll
        for (int c = 0; c < NPC; ++c) czf[c][v] = SPLIT_E ? zf : 1024.f / (float)(1 << code_exp<BITS>(c, 0)) + zf;
      }
    }
    f32x4 acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 xsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cu = 0; cu < GU; ++cu) {
      const int c = gi * GU + cu;
      const u32x4 araw = xrow[4 * c];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        uint32_t b[4];
        decode8<BITS, !BF>(word_at<VEC>(wv[c][0], v), NW > 1 ? word_at<VEC>(wv[c][NW - 1], v) : 0u, j, dm, b);
        if constexpr (BF) {
          uint32_t d[4];
          // A factor of 1 is kept opaque: the compiler would otherwise fold
          // fma(h, 1, c) into a conversion and an add, where the
          // mixed-precision FMA (v_fma_mix_f32) takes the fp16 half as is.
          float one = 1.f;
          asm("" : "+v"(one));
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const f16x2 h = as_f16x2(b[p]);
            const int pc = pair_class<BITS>(p);
            const float s_lo = code_exp<BITS>(p, 0) == 0 ? one : 1.0f / (float)(1 << code_exp<BITS>(p, 0));
            const float s_hi = code_exp<BITS>(p, 1) == 0 ? one : 1.0f / (float)(1 << code_exp<BITS>(p, 1));
            if constexpr (SPLIT_E) {
              d[p] = pack_bf16(__builtin_fmaf((float)h.x, s_lo, -1024.f * s_lo) - czf[pc][v],
                               __builtin_fmaf((float)h.y, s_hi, -1024.f * s_hi) - czf[pc][v]);
            } else {
              d[p] = pack_bf16(__builtin_fmaf((float)h.x, s_lo, -czf[pc][v]), __builtin_fmaf((float)h.y, s_hi, -czf[pc][v]));
            }
          }
          const bf16x8 A = __builtin_bit_cast(bf16x8, araw);
          const bf16x8 B = __builtin_bit_cast(bf16x8, u32x4{d[0], d[1], d[2], d[3]});
          acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[v], 0, 0, 0);
        } else {
          const f16x8 A = __builtin_bit_cast(f16x8, araw);
          acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pack8(b[0], b[1], b[2], b[3]), acc[v], 0, 0, 0);
        }
      }
      if constexpr (!BF && !XSUM_LDS) xsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, araw), ones, xsum, 0, 0, 0);
    }
    // One row: only element 0 (row 0) of the accumulators is used.
    constexpr int NE = M1 ? 1 : 4;
    if constexpr (BF) {
#pragma unroll
      for (int v = 0; v < VEC; ++v)
#pragma unroll
        for (int i = 0; i < NE; ++i) total[v][i] = __builtin_fmaf(sc[v], acc[v][i], total[v][i]);
    } else {
      // s 2^24 (acc - z 2^-24 sum x): both power-of-two factors are exact.
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float zq = half_bits_to_float(half_bits<VEC>(zraw[gi], v)) * 0x1p-24f;
        const float sq = sc[v] * 0x1p24f;
#pragma unroll
        for (int i = 0; i < NE; ++i)
          total[v][i] = __builtin_fmaf(sq, __builtin_fmaf(-zq, XSUM_LDS ? xsg[gi] : xsum[i], acc[v][i]), total[v][i]);
      }
    }
  }

  // ---- 4. the block's waves summed in wave order, in the LDS that held the
  // activations (hence the barrier first); bias; one rounding.
  // D layout: lane holds rows 4 j + i (i < 4) of column VEC * cl + v.
  __syncthreads();
  const int rows = M1 ? 1 : g.M;
  if constexpr (M1) {
    if (j == 0) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) red[wave * COLS + VEC * cl + v] = total[v][0];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * j + i;
      if (row < rows) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) red[(wave * rows + row) * COLS + VEC * cl + v] = total[v][i];
      }
    }
  }
  __syncthreads();
  const int entries = rows * COLS;
  for (int e = tid; e < entries; e += THREADS) {
    const int row = e / COLS, col = e - row * COLS;
    if (n0 + col < g.N) {
      float sum = red[e];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w * entries + e];
      if (g.bias) sum += bits_to_float<BF>(g.bias[n0 + col]);
      g.y[(size_t)row * g.N + n0 + col] = float_to_bits<BF>(sum);
    }
  }
}

template <int BITS, int VEC, int WAVES, int UPW, int GPW, bool BF>
hipError_t launch_wave_typed(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  const size_t lds = cmax(64 * WAVES * kWaveXPerThread * 16, WAVES * a.M * 16 * VEC * 4);
  const int grid = a.one_xcd > 1 ? p.nstrips * a.one_xcd : p.nstrips;
  if (a.M == 1) gemv_wave_kernel<BITS, VEC, WAVES, UPW, GPW, BF, true><<<grid, 64 * WAVES, lds, s>>>(a);
  else gemv_wave_kernel<BITS, VEC, WAVES, UPW, GPW, BF, false><<<grid, 64 * WAVES, lds, s>>>(a);
  return hipGetLastError();
}

// Weight words a lane holds: UPW * NW * VEC <= 32 (the plan only picks such shapes).
template <int BITS, int VEC, int UPW> constexpr bool wave_fits() { return UPW * Bits<BITS>::NW * VEC <= 32; }

template <int BITS, int VEC, int WAVES, int UPW, bool BF>
hipError_t launch_wave_if(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if constexpr (wave_fits<BITS, VEC, UPW>()) {
    switch (p.gpw) {
      case 1: return launch_wave_typed<BITS, VEC, WAVES, UPW, 1, BF>(p, a, s);
      case 2: return launch_wave_typed<BITS, VEC, WAVES, UPW, 2, BF>(p, a, s);
      case 4: if constexpr (UPW >= 4) return launch_wave_typed<BITS, VEC, WAVES, UPW, 4, BF>(p, a, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int BITS, int VEC, bool BF>
hipError_t launch_wave_vec(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if (p.waves == 8) {
    switch (p.upw) {
      case 2: return launch_wave_if<BITS, VEC, 8, 2, BF>(p, a, s);
      case 4: return launch_wave_if<BITS, VEC, 8, 4, BF>(p, a, s);
      case 8: return launch_wave_if<BITS, VEC, 8, 8, BF>(p, a, s);
      case 16: return launch_wave_if<BITS, VEC, 8, 16, BF>(p, a, s);
    }
  } else if (p.waves == 16) {
    switch (p.upw) {
      case 8: return launch_wave_if<BITS, VEC, 16, 8, BF>(p, a, s);
      case 16: return launch_wave_if<BITS, VEC, 16, 16, BF>(p, a, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int BITS, bool BF>
hipError_t launch_wave_bits(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if (p.vec == 1) return launch_wave_vec<BITS, 1, BF>(p, a, s);
  if (p.vec == 2) return launch_wave_vec<BITS, 2, BF>(p, a, s);
  return launch_wave_vec<BITS, 4, BF>(p, a, s);
}

}  // namespace
}  // namespace qmm
