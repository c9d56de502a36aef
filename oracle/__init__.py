"""CPU oracle (test infrastructure only; never imported by the GPU library)."""
from .lora_ref import *  # noqa: F401,F403
from .lora_ref import (bf16_bits_to_f64, bf16_rne_bits, decode_absmax_dq, decode_q4,
                       decode_q4_bits, decode_q4dq_bits, decode_q4_weight,
                       linear_bwd, linear_fwd, merged_weight, mlp_bwd, mlp_fwd,
                       rel_fro, rmsnorm_bwd, rmsnorm_fwd, scaling, sigmoid, swiglu,
                       swiglu_bwd,
                       trainable_params)
