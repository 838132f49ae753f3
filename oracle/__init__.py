"""fp64 CPU oracle of the MLA gather-decode step (test infrastructure only)."""
from .mla_oracle import (  # noqa: F401
    attention_core,
    bf16_round,
    dense_row_reader,
    front_fold,
    gather_keys,
    mla_gather_decode_step,
    output_projection,
    resolve_row,
    rms_norm,
    rope_interleaved,
    to_f64_inputs,
)
