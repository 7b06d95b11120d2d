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
//    one word row with a non-temporal buffer load (the row offset of a unit is
//    a scalar), since weights are streamed once.
//  * A block first requests its activations (already in the operand order of
//    the matrix cores, per row, unit and lane group) and its rows of scales
//    and zero points, then every wave requests its weight words. Loads
//    complete in order, so the block waits for the first two only, puts them
//    in LDS, and each unit is computed as soon as its own weight words arrive.
//  * Codes become halves with one bitfield insert into the mantissa of 1024.0
//    (exact). A code may sit 2^e places up in that mantissa (1024 + 2^e q),
//    which saves shifts; one packed fused multiply-add by 2^-e then subtracts
//    1024 2^-e + zero, exactly when the zero point is an integer; otherwise q
//    is formed first (exact) and the zero point subtracted after.
//  * The multiply-accumulate runs on the matrix cores: V_MFMA_F32_16X16X32_F16
//    with x as the 16 x 32 A operand (rows >= M repeat row 0 and are never
//    stored) and the dequantized codes as the 32 x 16 B operand. Lane group
//    j = l / 16 of the wave feeds 8 of the 32 k values of a "unit" (32
//    consecutive k), so a unit never straddles a group (group_size % 32 == 0)
//    and the fp32 accumulator of a group is multiplied by that group's scale
//    once (exact dequantized values up to the scale product).
//  * Waves of a block take consecutive K ranges of the same column strip and
//    are summed through LDS in wave order. Blocks along K write fp32 partial
//    sums; the last block of a strip to arrive (an atomic ticket) adds the
//    partials in split order and writes fp16 (round to nearest even). The sum
//    order never depends on arrival order, so results are bitwise repeatable,
//    and the ticket is reset to zero by that block.
#include "gemv_common.h"

namespace qmm {

hipError_t launch_gemv_wave_b1(const GemvPlan& p, const GemvArgs& a, bool bf16, hipStream_t s);
hipError_t launch_gemv_wave_b2(const GemvPlan& p, const GemvArgs& a, bool bf16, hipStream_t s);
hipError_t launch_gemv_wave_b3(const GemvPlan& p, const GemvArgs& a, bool bf16, hipStream_t s);
hipError_t launch_gemv_wave_b4(const GemvPlan& p, const GemvArgs& a, bool bf16, hipStream_t s);
hipError_t launch_gemv_wave_b8(const GemvPlan& p, const GemvArgs& a, bool bf16, hipStream_t s);

namespace {

constexpr int kMaxM = 16;
constexpr int kMaxSplit = 16;  // blocks along K per column strip
// Arrival counters live in a fixed header at the start of the workspace, one
// per column strip, and partial sums start after it. The header never
// overlaps any call's partial sums, so counters left at zero by one call are
// still zero for the next call, whatever the two shapes are.
constexpr size_t kCounterHeaderBytes = size_t(kGemvMaxStrips) * 4;

// LDS of a block: staged activations and scales / zero points, 9 KiB per
// wave (144 KiB for 16 waves, so that blocks of fewer waves can share a CU).
// The per-wave partial sums reuse the same space once every wave is done
// with the staged data.
constexpr int stage_bytes(int waves) { return waves * 9 * 1024; }
constexpr int kXPerThread = 4;  // activation slots one thread stages at most

// BF: bf16 data (x, scales, zero points, bias, y); the dequantized codes are
// then formed in fp32 and rounded once to bf16 for the bf16 matrix-core form.
template <int BITS, int VEC, int WAVES, bool BF>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(GemvArgs g) {
  constexpr int NW = Bits<BITS>::NW;
  constexpr int NPC = kPairClasses<BITS>;
  constexpr int CH = chunk_units<BITS, VEC, WAVES>();
  constexpr int COLS = 16 * VEC;
  constexpr int CP = COLS / 8;  // 16-byte pieces per staged row of scales or zero points
  constexpr int CP_LOG2 = VEC == 1 ? 1 : (VEC == 2 ? 2 : 3);
  constexpr int THREADS = 64 * WAVES;
  constexpr int kRedBytes = WAVES * kMaxM * COLS * 4;  // [WAVES][M][COLS] fp32
  __shared__ __attribute__((aligned(16))) unsigned char lds[cmax(stage_bytes(WAVES), kRedBytes)];
  float* red = reinterpret_cast<float*>(lds);
  __shared__ int wave_exact[WAVES];
  __shared__ int last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is the same for every lane of a wave; saying so keeps all
  // unit bookkeeping below in scalar registers and scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane >> 4;   // lane group: which 8 k of a unit
  const int cl = lane & 15;  // column group within the wave
  const int strip = xcd_strip(blockIdx.x, gridDim.x, g.xcd_log2);
  const int split = blockIdx.y;
  const int n0 = strip * COLS;
  const int nc = n0 + VEC * cl;  // first of this lane's VEC columns
  const int ncc = nc < g.N ? nc : 0;  // clamped: every load below is in bounds
  // A-operand row of this lane. Rows >= M read row 0: those MFMA rows only
  // produce outputs that are never stored.
  const int m = cl < g.M ? cl : 0;

  const int U = g.K / 32;
  const int ub0 = split * g.units_per_block;
  const int ub1 = min(U, ub0 + g.units_per_block);
  const int nub = ub1 - ub0;
  const int per_wave = (g.units_per_block + WAVES - 1) / WAVES;
  const int ua = min(ub1, ub0 + wave * per_wave);
  const int uz = min(ub1, ua + per_wave);
  auto group_of = [&](int u) { return g.upg_log2 >= 0 ? (u >> g.upg_log2) : u / g.upg; };
  const int gb0 = group_of(ub0);
  const int ngb = group_of(ub1 - 1) - gb0 + 1;  // groups this block touches
  const int G = U / g.upg;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(g.x, (size_t)g.M * g.K * 2);
  const long long wcols = plane_cols(g.N, g.strips);
  const int wrs = plane_row_stride(g.N, g.strips);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(g.qw, (size_t)U * unit_rows<BITS>(0) * wcols * 4);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(BITS == 3 ? g.qlo : g.qw, (size_t)U * unit_rows<BITS>(NW - 1) * wcols * 4);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.scales, (size_t)G * g.N * 2);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(g.zeros, (size_t)G * g.N * 2);

  // ---- 1. staging requests: activation slots (row, unit, lane group) of the
  // block's K range, and 16-byte pieces of its rows of scales and zero points.
  const int ubp_log2 = g.ubp_log2;
  u32x4 xraw[kXPerThread];
#pragma unroll
  for (int i = 0; i < kXPerThread; ++i) {
    const int sl = tid + THREADS * i;
    const int mm = sl >> (ubp_log2 + 2), uu = (sl >> 2) & ((1 << ubp_log2) - 1), jj = sl & 3;
    if (mm < g.M && uu < nub)
      xraw[i] = load_x_slot<BITS>(rx, (uint32_t)(mm * g.K + 32 * (ub0 + uu) + x_first<BITS>(jj)) * 2u);
  }
  const int sz_row = tid >> CP_LOG2, sz_cp = tid & (CP - 1);
  const bool sz_on = sz_row < ngb;
  u32x4 sraw = u32x4{0u, 0u, 0u, 0u}, zraw = u32x4{0u, 0u, 0u, 0u};
  if (sz_on) {
    const uint32_t voff = ((uint32_t)(gb0 + sz_row) * (uint32_t)g.N + (uint32_t)min(n0 + 8 * sz_cp, g.N - 8)) * 2u;
    sraw = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
    zraw = __builtin_amdgcn_raw_buffer_load_b128(rz, voff, 0, 0);
  }

  // ---- 2. weight words of the wave's first batch of units (the only stream
  // from HBM): per lane VEC adjacent columns of one word row per plane. Units
  // past the wave's range repeat its last unit and are not used.
  uint32_t woff[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w)
    woff[w] = (plane_col(ncc, U * unit_rows<BITS>(w), g.strips) + (uint32_t)(lane_row<BITS>(j, w) * wrs)) * 4u;
  typename Vec<VEC>::T wv[CH][NW];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int u = min(base + c, uz - 1);  // uz >= 1
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint32_t soff = (uint32_t)(u * unit_rows<BITS>(w)) * (uint32_t)wrs * 4u;
        wv[c][w] = load_words<VEC>((BITS == 3 && w == 1) ? rl : rw, woff[w], soff);
      }
    }
  };
  load_batch(ua);

  // ---- 3. staged data into LDS, waiting for the staging requests only. The
  // barrier also tells every wave whether all of the block's zero points are
  // integers (|z| <= 1024), for which one packed add dequantizes exactly.
  // Scales and zero points are staged ready for use, per (group row, column):
  // the fp32 scale; the fp16 pair (-z, -z); and per pair class c the fp16
  // pair -(1024 2^-e + z) (exact path) or, for bf16 data, fp32 1024 2^-e + z
  // (z alone for 1-bit codes, whose halves differ in e).
  constexpr bool SPLIT_E = BITS == 1;
  u32x4* xs = reinterpret_cast<u32x4*>(lds);
  const int xs_bytes = g.M << (ubp_log2 + 6);
  const int gstride = COLS << g.gp_log2;  // words per staged array
  float* s_sc = reinterpret_cast<float*>(lds + xs_bytes);       // [group row][COLS]
  uint32_t* s_zs = reinterpret_cast<uint32_t*>(s_sc + gstride);  // [group row][COLS]
  uint32_t* s_zc = s_zs + gstride;                               // [NPC][group row][COLS]
#pragma unroll
  for (int i = 0; i < kXPerThread; ++i) {
    const int sl = tid + THREADS * i;
    const int mm = sl >> (ubp_log2 + 2), uu = (sl >> 2) & ((1 << ubp_log2) - 1);
    if (mm < g.M && uu < nub) xs[sl] = x_operand<BITS>(xraw[i]);
  }
  bool exact = !BF;
  if (sz_on) {
    uint32_t scv[8], zsv[8], zcv[NPC][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t sb = (uint16_t)(sraw[e >> 1] >> (16 * (e & 1)));
      const uint16_t zb = (uint16_t)(zraw[e >> 1] >> (16 * (e & 1)));
      const float zf = bits_to_float<BF>(zb);
      scv[e] = __builtin_bit_cast(uint32_t, bits_to_float<BF>(sb));
      if constexpr (!BF) {
        exact = exact && (zf == __builtin_rintf(zf)) && (__builtin_fabsf(zf) <= 1024.f);
        const f16 nz = -__builtin_bit_cast(f16, zb);
        zsv[e] = as_u32(f16x2{nz, nz});
      }
#pragma unroll
      for (int c = 0; c < NPC; ++c) {
        const float base_lo = 1024.f / (float)(1 << code_exp<BITS>(c, 0));
        const float base_hi = 1024.f / (float)(1 << code_exp<BITS>(c, 1));
        if constexpr (BF) {
          zcv[c][e] = __builtin_bit_cast(uint32_t, SPLIT_E ? zf : base_lo + zf);
        } else {
          // exact when the zero point is an integer with |z| <= 1024 (1024 2^-e + z within 2048)
          zcv[c][e] = as_u32(f16x2{(f16)(-(base_lo + zf)), (f16)(-(base_hi + zf))});
        }
      }
    }
    const int o = sz_row * COLS + 8 * sz_cp;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint32_t*>(s_sc) + o + 4 * h) =
          u32x4{scv[4 * h], scv[4 * h + 1], scv[4 * h + 2], scv[4 * h + 3]};
      if constexpr (!BF)
        *reinterpret_cast<u32x4*>(s_zs + o + 4 * h) = u32x4{zsv[4 * h], zsv[4 * h + 1], zsv[4 * h + 2], zsv[4 * h + 3]};
#pragma unroll
      for (int c = 0; c < NPC; ++c)
        *reinterpret_cast<u32x4*>(s_zc + c * gstride + o + 4 * h) =
            u32x4{zcv[c][4 * h], zcv[c][4 * h + 1], zcv[c][4 * h + 2], zcv[c][4 * h + 3]};
    }
  }
  const bool wave_ok = __all(exact);
  if (lane == 0) wave_exact[wave] = wave_ok;
  __syncthreads();
  int all_ok = 1;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) all_ok &= wave_exact[w];
  const int zfast = __builtin_amdgcn_readfirstlane(all_ok);

  // ---- 4. the wave's units.
  const DecodeMasks<BITS> dm = decode_masks<BITS>();
  f32x4 total[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) total[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4* xrow = xs + (m << ubp_log2) * 4 + j;  // slot of unit u: xrow[4 (u - ub0)]

  auto run = [&](auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    // One accumulator per column, added into `total` times the group's scale
    // and cleared when the next group starts.
    f32x4 acc[VEC];
    float sc[VEC], czf[NPC][VEC];
    f16x2 zc[NPC][VEC], mz[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
      sc[v] = 0.f;
      mz[v] = f16x2{0, 0};
#pragma unroll
      for (int c = 0; c < NPC; ++c) { czf[c][v] = 0.f; zc[c][v] = f16x2{0, 0}; }
    }
    int cur_g = -1;
    auto chunk = [&](int base) {
      const u32x4* xb = xrow + 4 * (base - ub0);  // unit base + c at xb[4 c]
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int u = base + c;
        if (u >= uz) break;  // scalar
        const int grp = group_of(u);
        if (grp != cur_g) {  // scalar
          // A real branch: the group change is rare, and selecting its
          // results on every unit would cost more than the branch.
          asm volatile("" ::: "memory");
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            total[v] += sc[v] * acc[v];
            acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          cur_g = grp;
          const int o = (grp - gb0) * COLS + VEC * cl;
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            sc[v] = s_sc[o + v];
            if constexpr (!BF) mz[v] = as_f16x2(s_zs[o + v]);
#pragma unroll
            for (int c = 0; c < NPC; ++c) {
              if constexpr (BF) czf[c][v] = __builtin_bit_cast(float, s_zc[c * gstride + o + v]);
              else zc[c][v] = as_f16x2(s_zc[c * gstride + o + v]);
            }
          }
        }
        const u32x4 araw = xb[4 * c];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          uint32_t b[4];
          decode8<BITS>(word_at<VEC>(wv[c][0], v), NW > 1 ? word_at<VEC>(wv[c][NW - 1], v) : 0u, j, dm, b);
          uint32_t d[4];
          if constexpr (BF) {
            // A factor of 1 is kept opaque: the compiler would otherwise fold
            // fma(h, 1, c) into a conversion and an add, where the
            // mixed-precision FMA (v_fma_mix_f32) takes the fp16 half as is.
            float one = 1.f;
            asm("" : "+v"(one));
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const f16x2 h = as_f16x2(b[p]);
              const int c = pair_class<BITS>(p);
              const float s_lo = code_exp<BITS>(p, 0) == 0 ? one : 1.0f / (float)(1 << code_exp<BITS>(p, 0));
              const float s_hi = code_exp<BITS>(p, 1) == 0 ? one : 1.0f / (float)(1 << code_exp<BITS>(p, 1));
              if constexpr (SPLIT_E) {
                // q exactly, then one rounding of q - z
                d[p] = pack_bf16(__builtin_fmaf((float)h.x, s_lo, -1024.f * s_lo) - czf[c][v],
                                 __builtin_fmaf((float)h.y, s_hi, -1024.f * s_hi) - czf[c][v]);
              } else {
                d[p] = pack_bf16(__builtin_fmaf((float)h.x, s_lo, -czf[c][v]), __builtin_fmaf((float)h.y, s_hi, -czf[c][v]));
              }
            }
            const bf16x8 A = __builtin_bit_cast(bf16x8, araw);
            const bf16x8 B = __builtin_bit_cast(bf16x8, u32x4{d[0], d[1], d[2], d[3]});
            acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[v], 0, 0, 0);
          } else {
            if constexpr (FAST) {
#pragma unroll
              for (int p = 0; p < 4; ++p)
                d[p] = as_u32(scale_add<BITS>(p, as_f16x2(b[p]), zc[pair_class<BITS>(p)][v]));
            } else {
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                const f16x2 s = pair_scale<BITS>(p);
                const f16x2 q = scale_add<BITS>(p, as_f16x2(b[p]), f16x2{(f16)(-1024.f) * s.x, (f16)(-1024.f) * s.y});
                d[p] = as_u32(q + mz[v]);
              }
            }
            const f16x8 A = __builtin_bit_cast(f16x8, araw);
            const f16x8 B = pack8(d[0], d[1], d[2], d[3]);
            acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, acc[v], 0, 0, 0);
          }
        }
      }
    };
    chunk(ua);  // its words were requested before the staging barrier
    for (int base = ua + CH; base < uz; base += CH) {
      load_batch(base);
      chunk(base);
    }
    {
#pragma unroll
      for (int v = 0; v < VEC; ++v) total[v] += sc[v] * acc[v];
    }
  };
  if (zfast) run(std::integral_constant<bool, true>{});
  else run(std::integral_constant<bool, false>{});

  // ---- 5. the block's waves are summed in wave order, in LDS that held
  // the staged data (hence the barrier first).
  __syncthreads();
  // D layout: lane holds rows 4 j + i (i < 4) of column VEC * cl + v.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * j + i;
    if (row < g.M) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) red[(wave * g.M + row) * COLS + VEC * cl + v] = total[v][i];
    }
  }
  __syncthreads();

  const int entries = g.M * COLS;
  auto block_sum = [&](int e) {
    float sum = red[e];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w * entries + e];
    return sum;
  };
  // The bias joins the fp32 sum before its one rounding to fp16.
  auto bias_at = [&](int n) { return g.bias ? bits_to_float<BF>(g.bias[n]) : 0.f; };
  if (g.ksplit == 1) {
    for (int e = tid; e < entries; e += THREADS) {
      const int row = e / COLS, col = e - row * COLS;
      if (n0 + col < g.N)
        g.y[(size_t)row * g.N + n0 + col] = float_to_bits<BF>(block_sum(e) + bias_at(n0 + col));
    }
    return;
  }

  // Blocks along K hand over through the workspace, in the pattern of a
  // ticketed reduction: every thread publishes its partial sums (device-scope
  // atomic stores) and then issues a release fence at device scope; the block
  // meets at a barrier, after which one thread takes the strip's ticket with
  // an acquire-release read-modify-write. The block that draws the last
  // ticket therefore follows every other block's release, and each of its
  // threads issues an acquire fence before reading the partials.
  float* mypart = g.part + (size_t)split * g.M * g.N;
  for (int e = tid; e < entries; e += THREADS) {
    const int row = e / COLS, col = e - row * COLS;
    if (n0 + col < g.N)
      __hip_atomic_store(mypart + (size_t)row * g.N + n0 + col, block_sum(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&g.counters[strip], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last_flag = (prev == (uint32_t)(g.ksplit - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int e = tid; e < entries; e += THREADS) {
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
      float sum = pv[0];
#pragma unroll
      for (int sp = 1; sp < kMaxSplit; ++sp) sum += (sp < g.ksplit) ? pv[sp] : 0.f;
      g.y[off] = float_to_bits<BF>(sum + bias_at(n0 + col));
    }
  }
  if (tid == 0) __hip_atomic_store(&g.counters[strip], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, int VEC, int WAVES, bool BF>
hipError_t launch_typed(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  dim3 grid(p.nstrips, p.ksplit);
  gemv_kernel<BITS, VEC, WAVES, BF><<<grid, 64 * WAVES, 0, s>>>(a);
  return hipGetLastError();
}

// The plan uses 16 waves per block, and 8 for 4 columns per lane at 3 or 8
// bits; other wave counts are tuning options.
template <int BITS, bool BF>
hipError_t launch_bits(const GemvPlan& p, const GemvArgs& a, hipStream_t s) {
  if (p.vec == 1) return p.waves == 16 ? launch_typed<BITS, 1, 16, BF>(p, a, s) : launch_typed<BITS, 1, 8, BF>(p, a, s);
  if (p.waves == 16) return p.vec == 2 ? launch_typed<BITS, 2, 16, BF>(p, a, s) : launch_typed<BITS, 4, 16, BF>(p, a, s);
  if (p.waves == 8) return p.vec == 2 ? launch_typed<BITS, 2, 8, BF>(p, a, s) : launch_typed<BITS, 4, 8, BF>(p, a, s);
  return p.vec == 2 ? launch_typed<BITS, 2, 4, BF>(p, a, s) : launch_typed<BITS, 4, 4, BF>(p, a, s);
}

template <bool BF>
hipError_t launch_dtype(const GemvPlan& p, const GemvArgs& a, int bits, hipStream_t s) {
  switch (bits) {
    case 1: return launch_bits<1, BF>(p, a, s);
    case 2: return launch_bits<2, BF>(p, a, s);
    case 3: return launch_bits<3, BF>(p, a, s);
    case 4: return launch_bits<4, BF>(p, a, s);
    case 8: return launch_bits<8, BF>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wave_any(const GemvPlan& p, const GemvArgs& a, int bits, bool bf16, hipStream_t s) {
  switch (bits) {
    case 1: return launch_gemv_wave_b1(p, a, bf16, s);
    case 2: return launch_gemv_wave_b2(p, a, bf16, s);
    case 3: return launch_gemv_wave_b3(p, a, bf16, s);
    case 4: return launch_gemv_wave_b4(p, a, bf16, s);
    case 8: return launch_gemv_wave_b8(p, a, bf16, s);
    default: return hipErrorInvalidValue;
  }
}

int ceil_log2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

}  // namespace

GemvPlan gemv_plan(int M, int K, int N, int bits, int group_size, DeviceTopo topo) {
  GemvPlan p{};
  const int cus = topo.cus > 0 ? topo.cus : 256;
  p.xcds = topo.xcds > 0 ? topo.xcds : 8;
  // Narrowest column strip whose blocks fit in one round on the CUs (16, 32
  // or 64 columns per wave).
  int vec = 4;
  if ((N + 15) / 16 <= cus) vec = 1;
  else if ((N + 31) / 32 <= cus) vec = 2;
  if (QMM_GEMV_VEC != 0) vec = QMM_GEMV_VEC;
  p.vec = vec;
  p.strip_cols = 16 * vec;
  p.nstrips = (N + p.strip_cols - 1) / p.strip_cols;
  const int U = K / 32;
  const int nw = bits == 3 || bits == 8 ? 2 : 1;  // words per lane per unit and column
  // 16 waves per block, except where two words per lane per unit (3-bit,
  // 8-bit) at 4 columns per lane need more registers than 16 waves allow.
  p.waves = (vec == 4 && (bits == 3 || bits == 8)) ? 8 : 16;
  if (QMM_GEMV_WAVES != 0) p.waves = QMM_GEMV_WAVES;
  p.upg = group_rows(K, group_size) / 32;
  p.upg_log2 = -1;
  for (int l = 0; l < 31; ++l)
    if ((1 << l) == p.upg) p.upg_log2 = l;
  const long long per_split = (long long)p.nstrips * p.waves;
  int ks = (int)((QMM_GEMV_TARGET_WAVES + per_split - 1) / per_split);
  int max_ks = U / p.waves;  // at least one unit per wave
  max_ks = max_ks < 1 ? 1 : (max_ks > kMaxSplit ? kMaxSplit : max_ks);
  ks = ks < 1 ? 1 : (ks > max_ks ? max_ks : ks);

  // The wave kernel: one block per strip over all of K (where no split along
  // K is wanted), U = waves * upw with 8 waves (else 16), at most 32 weight
  // words per lane, groups of a power-of-two number of units (or one group),
  // at most 4 groups per wave, and the block's activations within its
  // staging area (4 slots per thread, 64 KiB).
  if (ks == 1 && QMM_GEMV_WAVES == 0) {
    const bool one_group = group_size == -1;
    const int gl = one_group ? 30 : p.upg_log2;
    for (int w : {8, 16}) {
      if (U % w) continue;
      const int upw = U / w;
      const bool upw_ok = (w == 8 && (upw == 2 || upw == 4 || upw == 8 || upw == 16)) ||
                          (w == 16 && (upw == 8 || upw == 16));
      if (!upw_ok || upw * nw * vec > 32 || gl < 0) continue;
      // groups per wave: 1 when a group holds all of the wave's units
      // (upw is a power of two, so a group of >= upw units aligns with it)
      const int gpw = (one_group || p.upg >= upw) ? 1 : upw / p.upg;
      const long long rbytes = (long long)w * M * 16 * vec * 4;
      if (gpw > 4 || (long long)M * U * 4 > 4LL * 64 * w || rbytes > 65536) continue;
      p.kind = 1;
      p.waves = w;
      p.upw = upw;
      p.gl = gl;
      p.gpw = gpw;
      p.ksplit = 1;
      p.units_per_block = U;
      // Strips that fit on one XCD's CUs, with at most 1 MiB of weight
      // words, all run on XCD 0, which starts its blocks first (one XCD's
      // share of the memory system then carries them).
      const long long wbytes = (long long)K * N * bits / 8;
      p.one_xcd = (QMM_GEMV_ONE_XCD && p.xcds > 1 && p.nstrips <= cus / p.xcds && wbytes <= (1LL << 20)) ? p.xcds : 0;
      p.valid = 1;
      return p;
    }
  }

  // Otherwise the split kernel: blocks along K are added when the strips
  // alone leave too few waves in flight, or when a block's activations and
  // scales / zero points would not fit its staging area.
  const int threads = 64 * p.waves, cols = p.strip_cols;
  for (;; ++ks) {
    if (ks > kMaxSplit) return GemvPlan{};  // no valid plan: valid == 0
    const int upb = (U + ks - 1) / ks;
    const int ubp_log2 = ceil_log2(upb);
    int groups = 0;  // most groups one block touches
    for (int s = 0; s * upb < U; ++s) {
      const int u0 = s * upb, u1 = (U < u0 + upb ? U : u0 + upb) - 1;
      const int gcount = u1 / p.upg - u0 / p.upg + 1;
      groups = gcount > groups ? gcount : groups;
    }
    const int gp_log2 = ceil_log2(groups);
    const long long x_slots = (long long)M << (ubp_log2 + 2);
    const int npc = bits == 1 ? 4 : ((bits == 2 || bits == 4) ? 2 : 1);
    const long long stage = (x_slots << 4) + (1LL << gp_log2) * cols * 4 * (2 + npc);
    if (x_slots <= (long long)kXPerThread * threads && ((long long)(cols / 8) << gp_log2) <= threads &&
        stage <= stage_bytes(p.waves)) {
      p.units_per_block = upb;
      p.ubp_log2 = ubp_log2;
      p.gp_log2 = gp_log2;
      break;
    }
  }
  p.ksplit = (U + p.units_per_block - 1) / p.units_per_block;
  if (p.ksplit > 1) {
    p.counters_bytes = kCounterHeaderBytes;
    p.workspace_bytes = p.counters_bytes + (size_t)p.ksplit * M * N * sizeof(float);
  }
  p.valid = 1;
  return p;
}

hipError_t launch_gemv(const GemvPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                       const uint32_t* qlo, const uint16_t* zeros, const uint16_t* scales,
                       const uint16_t* bias, int N, int bits, int group_size, uint16_t* y,
                       void* workspace, bool bf16, bool strips, hipStream_t s) {
  if (!p.valid) return hipErrorInvalidValue;
  GemvArgs a;
  a.x = x;
  a.qw = qw;
  a.qlo = qlo;
  a.zeros = zeros;
  a.scales = scales;
  a.bias = bias;
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
  a.ubp_log2 = p.ubp_log2;
  a.gp_log2 = p.gp_log2;
  a.xcd_log2 = -1;
  for (int l = 1; l < 8; ++l)
    if ((1 << l) == p.xcds && p.nstrips % p.xcds == 0) a.xcd_log2 = l;
  a.gl = p.gl;
  a.strips = strips ? 1 : 0;
  a.one_xcd = p.kind == 1 ? p.one_xcd : 0;
  if (p.kind == 1) return launch_wave_any(p, a, bits, bf16, s);
  return bf16 ? launch_dtype<true>(p, a, bits, s) : launch_dtype<false>(p, a, bits, s);
}

}  // namespace qmm
