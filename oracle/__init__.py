"""fp64 CPU oracle of the spatial self-attention block (test infrastructure only)."""
from .ssa_oracle import (  # noqa: F401
    EPS, PARAM_KEYS, attention, check_args, forward, forward_pixels,
    forward_stages, group_norm, image, linear, softmax_keys, tokens,
)
