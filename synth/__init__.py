"""Seeded synthetic inputs shared by the fp64 oracle and the HIP path.

This package draws random tensors and rounds them to bfloat16; it holds none of the
tensor-parallel arithmetic. Both the oracle (``oracle/``) and the HIP library
(``tensor_transformer_layers_amd``) are fed from here, and neither imports the other.
"""
from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_round,
    bf16_bits,
    attn_inputs,
    gqa_inputs,
    layernorm_params,
    mlp_inputs,
    swiglu_inputs,
    normal_matrix,
    partials_inputs,
    sample_rows,
)
