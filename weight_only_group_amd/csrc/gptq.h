// Launchers of the GPTQModel-format conversions (gptq.hip), called by the C ABI.
#pragma once

#include "common.h"

namespace qmm {

int gptq_values_per_word(int bits);  // 16, 10, 8, 4 for 2, 3, 4, 8 bits
hipError_t launch_unpack_qzeros(const uint32_t* qzeros, int G, int N, int bits, uint16_t* zeros, bool bf16,
                                hipStream_t stream);
hipError_t launch_repack_3bit10(const uint32_t* w10, int K, int N, uint32_t* plane2, uint32_t* plane1,
                                hipStream_t stream);

}  // namespace qmm
