// The wave-local decode product for 4-bit codes (instances of gemv_wave.h).
#include "gemv_wave.h"

namespace qmm {

hipError_t launch_gemv_wave_b4(const GemvPlan& p, const GemvArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_wave_bits<4, true>(p, a, s) : launch_wave_bits<4, false>(p, a, s);
}

}  // namespace qmm
