"""CPU oracle for the 4-bit-weight GEMM path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the benchmark's CPU-baseline leg, never by the library.  See
``oracle/w4_oracle.py`` for the definitions it follows.
"""
from . import formats  # noqa: F401
from . import w4_oracle  # noqa: F401
from .w4_oracle import (  # noqa: F401
    nibbles, weight_values, pb_v1_position, prepack_B, unprepack_B, exllama_to_logical,
    prepack_B_from_exllama,
    quant_act_per_token, quant_act_per_tensor, rmsnorm_rows, rmsnorm_quant_per_token, activation_integers, w4a8_group_partials, w4a8_gemm,
    zero_point_weights,
    w4a16_gemm, w4a16_gemm_prescaled_zeros, w4a16_group_partials,
)
