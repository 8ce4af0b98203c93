"""fp64 CPU oracle of the spatial self-attention block (test infrastructure only)."""
from .ssa_oracle import (  # noqa: F401
    BIAS_KEYS, EPS, PARAM_KEYS, attend, attention, check_args, check_options, forward,
    forward_pixels, forward_stages, group_norm, image, linear, merge_heads, qk_norm,
    rel_pos_bias, rope, rope_angles, softmax_keys, split_heads, tokens,
)
