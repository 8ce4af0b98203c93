"""MI355X (gfx950) spatial self-attention block.

    out = x + image(MHA(tokens(GN(x))))

(tensortonic problem "Spatial Self-Attention": GroupNorm, pixel tokens, Q/K/V
projections with biases, per-head softmax(Q_j K_j^T / sqrt(d)) V_j,
concatenated heads, output projection, residual in image layout.)

The computation runs in libssa.so's HIP kernels behind the C ABI in
include/ssa.h; this module only moves pointers.  torch supplies device memory
and the current stream.
"""
from __future__ import annotations

import torch

from ._binding import (  # noqa: F401
    BIAS_KEYS, EXPORTS, LIB_PATH, PARAM_ORDER, SSA_BF16, SSA_F32, STAGES, Options, SSAError,
    SSAValueError, lib, ssa_forward, ssa_forward_ex, ssa_forward_noalloc, ssa_forward_stage,
    ssa_forward_stage_ex, ssa_get_workspace_layout, ssa_noalloc_max_workspace, ssa_status_string,
    ssa_uses_fused_stage, ssa_workspace_size,
)
from ._binding import _raise

_DTYPES = {torch.float32: SSA_F32, torch.bfloat16: SSA_BF16}


def dtype_code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPES:
        raise SSAValueError(4, f"dtype {dtype}")
    return _DTYPES[dtype]


def _ptr(t) -> int:
    return 0 if t is None or t.numel() == 0 else t.data_ptr()


def _check_tensors(x: torch.Tensor, params: dict):
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor (the block runs only in the HIP kernels)")
    if x.dim() != 4:
        raise ValueError("x must be (B, C, H, W)")
    if set(params) != set(PARAM_ORDER):
        raise ValueError(f"params must have exactly the keys {PARAM_ORDER}")
    C = x.shape[1]
    for k in PARAM_ORDER:
        p = params[k]
        if p is None and k in BIAS_KEYS:
            continue  # a projection without a bias
        want = (C,) if (k.endswith("_bias") or k.startswith("norm")) else (C, C)
        if tuple(p.shape) != want:
            raise ValueError(f"{k} must have shape {want}, got {tuple(p.shape)}")
        if p.dtype != x.dtype or p.device != x.device:
            raise ValueError(f"{k} must match x's dtype and device")
        if not p.is_contiguous():
            raise ValueError(f"{k} must be contiguous")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (NCHW)")


def workspace_for(x: torch.Tensor, num_groups: int, num_heads: int) -> torch.Tensor:
    """A workspace tensor (uint8) of ssa_workspace_size bytes on x's device."""
    B, C, H, W = x.shape
    n = ssa_workspace_size(B, C, H, W, num_groups, num_heads, dtype_code(x.dtype))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=x.device)


def make_options(x, num_heads, rel_pos_table=None, q_norm_gamma=None, k_norm_gamma=None,
                 rope=False):
    """An Options structure for the optional steps, or None when none is on.

    rel_pos_table ((2H-1)(2W-1), num_heads), q_norm_gamma / k_norm_gamma
    (num_heads, d), all of x's dtype and device and contiguous; rope a bool.
    The tensors must stay alive until the call's kernels have run."""
    if rel_pos_table is None and q_norm_gamma is None and k_norm_gamma is None and not rope:
        return None
    B, C, H, W = x.shape
    d = C // num_heads
    for name, t, want in (("rel_pos_table", rel_pos_table, ((2 * H - 1) * (2 * W - 1), num_heads)),
                          ("q_norm_gamma", q_norm_gamma, (num_heads, d)),
                          ("k_norm_gamma", k_norm_gamma, (num_heads, d))):
        if t is None:
            continue
        if tuple(t.shape) != want:
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
        if t.dtype != x.dtype or t.device != x.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous with x's dtype and device")
    return Options(_ptr(rel_pos_table), _ptr(q_norm_gamma), _ptr(k_norm_gamma), 1 if rope else 0)


def forward_stages(x, num_groups: int, num_heads: int, options=None) -> tuple:
    """The stage names ssa_forward (ssa_forward_ex with `options`) runs for
    x's problem, in order."""
    B, C, H, W = x.shape
    if options is None and ssa_uses_fused_stage(B, C, H, W, num_groups, num_heads,
                                                dtype_code(x.dtype)):
        return ("gn_stats", "qkv_attention", "out_proj")
    return ("gn_stats", "qkv", "attention", "out_proj")


def forward_into(x, params, num_groups, num_heads, out, workspace, stage=None,
                 stream=None, options=None) -> None:
    """Enqueue the block (or one stage of it) on `stream` (default: torch's current).

    options: an Options structure (make_options) for ssa_forward_ex, or None."""
    _check_tensors(x, params)
    B, C, H, W = x.shape
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    ptrs = [_ptr(params[k]) for k in PARAM_ORDER]
    head = (_ptr(x), _ptr(out), ptrs, B, C, H, W, num_groups, num_heads, dtype_code(x.dtype))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), stream.cuda_stream)
    if stage is not None and options is not None:
        _raise(ssa_forward_stage_ex(STAGES.get(stage, stage), *head, options, *tail),
               "ssa_forward_stage_ex")
    elif stage is not None:
        _raise(ssa_forward_stage(STAGES.get(stage, stage), *head, *tail), "ssa_forward_stage")
    elif options is not None:
        _raise(ssa_forward_ex(*head, options, *tail), "ssa_forward_ex")
    else:
        _raise(ssa_forward(*head, *tail), "ssa_forward")


def spatial_self_attention(x: torch.Tensor, params: dict, num_groups: int, num_heads: int,
                           *, rel_pos_table=None, q_norm_gamma=None, k_norm_gamma=None,
                           rope: bool = False) -> torch.Tensor:
    """out = x + image(MHA(tokens(GN(x)))), shape and dtype of x.

    params holds the ten tensors norm_weight, norm_bias (C,), q/k/v/out_weight
    (C, C) stored (out, in), q/k/v/out_bias (C,), all of x's dtype; a bias may
    be None (a projection without a bias).  The keyword options switch on the
    optional steps of include/ssa.h's ssa_options: a 2-D relative-position
    bias table, per-head query/key normalisation gammas, rotary embeddings.
    """
    _check_tensors(x, params)
    opts = make_options(x, num_heads, rel_pos_table, q_norm_gamma, k_norm_gamma, rope)
    out = torch.empty_like(x)
    ws = workspace_for(x, num_groups, num_heads)
    forward_into(x, params, num_groups, num_heads, out, ws, options=opts)
    return out
