"""CPU oracle (test infrastructure only; see ``qmm_oracle``)."""
from .qmm_oracle import *  # noqa: F401,F403
from .qmm_oracle import (  # noqa: F401
    ABS_TOL, PLANE_BITS, REL_TOL, REL_TOL_BF16, SUPPORTED_BITS, bf16_to_f64, count_out_of_range, dequantize,
    dequantize_bf16, dequantize_fp16, elements_per_word, f64_to_bf16,
    group_rows, matmul, matmul_triple_loop, num_groups, pack, pack_3bit, pack_kmajor, parity_bound, parity_report,
    quantized_matmul, quantized_matmul_codes, unpack, unpack_3bit, unpack_kmajor,
    STRIP_COLS, to_strips, from_strips,
)
