"""CPU oracle (test infrastructure only; see mxfp4_oracle's header)."""
from .mxfp4_oracle import *  # noqa: F401,F403
from .mxfp4_oracle import (GROUP, E2M1_VALUES, E2M1_EMAX, C_NORM, sylvester_hadamard, fwht32,
                           transform, transform_dense_fp64, e8m0_scale, e2m1_nearest,
                           quantize_mxfp4, unpack_codes, dequantize_mxfp4, as_f32,
                           expert_of_rows, quant_act, weight_reciprocal, prepare_weights,
                           gemm, linear, within_tolerance, round_bf16, swiglu, swiglu_bound,
                           encode_groups, pack_codes, hessian, diagonal_blocks,
                           dequantize_groups, hessian_error, search_exponents,
                           prepare_weights_hessian, E2M1_LEVELS, code_levels, level_code,
                           flip_refine, layer_loss)
