// The wave-local decode product for 3-bit codes (instances of gemv_wave.h).
#include "gemv_wave.h"

namespace qmm {

hipError_t launch_gemv_wave_b3(const GemvPlan& p, const GemvArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch_wave_bits<3, true>(p, a, s) : launch_wave_bits<3, false>(p, a, s);
}

}  // namespace qmm
