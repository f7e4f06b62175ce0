"""fp64 CPU oracle (test infrastructure only; see ffn_oracle)."""
from .ffn_oracle import (  # noqa: F401
    as_f64, bf16_to_f64, f16_to_f64, silu, rmsnorm, swiglu_block,
    swiglu_block_intermediates, q8_dequant, swiglu_block_q8, block_from_stored,
    rmsnorm_from_stored,
)
