"""CPU oracle for the fused W4 base + sparse 4-bit residual linear.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg are its only users. The HIP library never imports, links or
runs anything from here, and this package imports nothing from the library.
"""
from .mosaic import (  # noqa: F401
    QMAX, SUPPORTED_GROUPS, MAX_K, OracleInputError, TOL_REL, TOL_ABS,
    to_fp16_rne, to_fp32_rne, check_inputs, base_scales, base_codes, base_error,
    budget, select_topk, residual_scales, residual_codes, pack_nibbles,
    unpack_nibbles, pack, dequant, linear, within_tolerance,
)
