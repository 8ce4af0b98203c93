"""ctypes binding of libssa.so (include/ssa.h).

Argument marshalling only: every step of the block runs in the library's HIP
kernels.  torch provides device memory and the current stream.  There is no
fallback: when libssa.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libssa.so")

SSA_OK = 0
STATUS_NAMES = {
    0: "SSA_OK", 1: "SSA_E_NULL", 2: "SSA_E_SHAPE", 3: "SSA_E_CONSTRAINT",
    4: "SSA_E_DTYPE", 5: "SSA_E_UNSUPPORTED", 6: "SSA_E_WORKSPACE",
    7: "SSA_E_ALIAS", 8: "SSA_E_ALIGN", 9: "SSA_E_HIP", 10: "SSA_E_STAGE",
    11: "SSA_E_SCRATCH",
}
SSA_F32, SSA_BF16 = 0, 1
STAGES = {"gn_stats": 0, "qkv": 1, "attention": 2, "out_proj": 3, "qkv_attention": 4}

# Parameter order of the ABI (the problem's parameter table).
PARAM_ORDER = (
    "norm_weight", "norm_bias",
    "q_weight", "k_weight", "v_weight", "out_weight",
    "q_bias", "k_bias", "v_bias", "out_bias",
)

EXPORTS = ("ssa_workspace_size", "ssa_get_workspace_layout", "ssa_forward",
           "ssa_forward_ex", "ssa_forward_stage", "ssa_forward_stage_ex", "ssa_forward_noalloc",
           "ssa_noalloc_max_workspace", "ssa_uses_fused_stage", "ssa_status_string")

BIAS_KEYS = ("q_bias", "k_bias", "v_bias", "out_bias")


class Options(ctypes.Structure):
    """ssa_options (include/ssa.h)."""
    _fields_ = [
        ("rel_pos_table", ctypes.c_void_p),
        ("q_norm_gamma", ctypes.c_void_p),
        ("k_norm_gamma", ctypes.c_void_p),
        ("rope", ctypes.c_int32),
    ]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [
        ("total", ctypes.c_size_t),
        ("gn_partial", ctypes.c_size_t),
        ("gn_stats", ctypes.c_size_t),
        ("gn_coef", ctypes.c_size_t),
        ("q", ctypes.c_size_t),
        ("k", ctypes.c_size_t),
        ("vt", ctypes.c_size_t),
        ("o", ctypes.c_size_t),
        ("rope", ctypes.c_size_t),
        ("qk32", ctypes.c_size_t),
        ("attn_part", ctypes.c_size_t),
        ("gn_splits", ctypes.c_int64),
        ("t_pad", ctypes.c_int64),
        ("d_pad", ctypes.c_int64),
    ]


class SSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


class SSAValueError(SSAError, ValueError):
    """Argument, shape, constraint or dtype errors."""


_lib = None


def lib() -> ctypes.CDLL:
    """Load libssa.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m spatial_self_attention_amd.build` "
            "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.ssa_workspace_size.restype = sz
    L.ssa_workspace_size.argtypes = [i64] * 6 + [ctypes.c_int]
    L.ssa_get_workspace_layout.restype = ctypes.c_int
    L.ssa_get_workspace_layout.argtypes = [i64] * 6 + [ctypes.c_int, ctypes.POINTER(WorkspaceLayout)]
    fwd = [vp] * 12 + [i64] * 6 + [ctypes.c_int, vp, sz, vp]
    L.ssa_forward.restype = ctypes.c_int
    L.ssa_forward.argtypes = fwd
    L.ssa_forward_stage.restype = ctypes.c_int
    L.ssa_forward_stage.argtypes = [ctypes.c_int] + fwd
    L.ssa_forward_ex.restype = ctypes.c_int
    L.ssa_forward_ex.argtypes = fwd[:19] + [ctypes.POINTER(Options)] + fwd[19:]
    L.ssa_forward_stage_ex.restype = ctypes.c_int
    L.ssa_forward_stage_ex.argtypes = [ctypes.c_int] + fwd[:19] + [ctypes.POINTER(Options)] + fwd[19:]
    L.ssa_forward_noalloc.restype = ctypes.c_int
    L.ssa_forward_noalloc.argtypes = fwd[:19] + [vp]
    L.ssa_noalloc_max_workspace.restype = sz
    L.ssa_noalloc_max_workspace.argtypes = []
    L.ssa_uses_fused_stage.restype = ctypes.c_int
    L.ssa_uses_fused_stage.argtypes = [i64] * 6 + [ctypes.c_int]
    L.ssa_status_string.restype = ctypes.c_char_p
    L.ssa_status_string.argtypes = [ctypes.c_int]
    _lib = L
    return L


def status_string(status: int) -> str:
    return ssa_status_string(status)


def _raise(status: int, where: str):
    if status == SSA_OK:
        return
    if status in (1, 2, 3, 4, 5, 6, 7, 8, 10, 11):
        raise SSAValueError(status, where)
    raise SSAError(status, where)


# --- same-name wrappers of the C entry points ------------------------------

def ssa_status_string(status: int) -> str:
    return lib().ssa_status_string(int(status)).decode()


def ssa_workspace_size(B, C, H, W, num_groups, num_heads, dtype) -> int:
    return int(lib().ssa_workspace_size(B, C, H, W, num_groups, num_heads, int(dtype)))


def ssa_get_workspace_layout(B, C, H, W, num_groups, num_heads, dtype) -> dict:
    lay = WorkspaceLayout()
    st = lib().ssa_get_workspace_layout(B, C, H, W, num_groups, num_heads, int(dtype),
                                        ctypes.byref(lay))
    _raise(st, "ssa_get_workspace_layout")
    return {name: int(getattr(lay, name)) for name, _ in WorkspaceLayout._fields_}


def ssa_forward(x_ptr, out_ptr, param_ptrs, B, C, H, W, num_groups, num_heads, dtype,
                ws_ptr, ws_bytes, stream_ptr) -> int:
    """Raw call: integer device pointers in, status code out."""
    return int(lib().ssa_forward(x_ptr, out_ptr, *param_ptrs, B, C, H, W, num_groups,
                                 num_heads, int(dtype), ws_ptr, ws_bytes, stream_ptr))


def ssa_forward_ex(x_ptr, out_ptr, param_ptrs, B, C, H, W, num_groups, num_heads, dtype,
                   options, ws_ptr, ws_bytes, stream_ptr) -> int:
    """Raw call with an Options structure (or None: the plain block)."""
    opt = ctypes.byref(options) if options is not None else None
    return int(lib().ssa_forward_ex(x_ptr, out_ptr, *param_ptrs, B, C, H, W, num_groups,
                                    num_heads, int(dtype), opt, ws_ptr, ws_bytes, stream_ptr))


def ssa_forward_stage(stage, x_ptr, out_ptr, param_ptrs, B, C, H, W, num_groups, num_heads,
                      dtype, ws_ptr, ws_bytes, stream_ptr) -> int:
    return int(lib().ssa_forward_stage(int(stage), x_ptr, out_ptr, *param_ptrs, B, C, H, W,
                                       num_groups, num_heads, int(dtype), ws_ptr, ws_bytes,
                                       stream_ptr))


def ssa_forward_stage_ex(stage, x_ptr, out_ptr, param_ptrs, B, C, H, W, num_groups, num_heads,
                         dtype, options, ws_ptr, ws_bytes, stream_ptr) -> int:
    """Raw call of one stage with an Options structure (or None)."""
    opt = ctypes.byref(options) if options is not None else None
    return int(lib().ssa_forward_stage_ex(int(stage), x_ptr, out_ptr, *param_ptrs, B, C, H, W,
                                          num_groups, num_heads, int(dtype), opt, ws_ptr,
                                          ws_bytes, stream_ptr))


def ssa_forward_noalloc(x_ptr, out_ptr, param_ptrs, B, C, H, W, num_groups, num_heads, dtype,
                        stream_ptr) -> int:
    """Raw call of the entry point that allocates nothing (the library's static
    scratch is the workspace): integer device pointers in, status code out."""
    return int(lib().ssa_forward_noalloc(x_ptr, out_ptr, *param_ptrs, B, C, H, W, num_groups,
                                         num_heads, int(dtype), stream_ptr))


def ssa_noalloc_max_workspace() -> int:
    return int(lib().ssa_noalloc_max_workspace())


def ssa_uses_fused_stage(B, C, H, W, num_groups, num_heads, dtype) -> bool:
    """Whether ssa_forward runs stages 0, 4, 3 (the fused kernel) for this problem."""
    return bool(lib().ssa_uses_fused_stage(B, C, H, W, num_groups, num_heads, int(dtype)))
