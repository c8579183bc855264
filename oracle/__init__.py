"""CPU oracle (test infrastructure only; see verify_oracle)."""

from .verify_oracle import (  # noqa: F401
    ancestor_mask,
    as_f64,
    bf16_bits_to_f64,
    default_scale,
    masked_attention,
    protected_set,
    select_row,
    select_verify_set,
    verify_attention,
)
