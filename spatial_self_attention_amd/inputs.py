"""Seeded synthetic inputs for the spatial self-attention block.

This module only draws numbers.  It holds none of the block's arithmetic, so
both the GPU path's tests/benchmark and the fp64 CPU oracle can take their
inputs from it without sharing any computation.

Workloads (shapes and value distributions) follow the five configurations the
block is measured on; the parameter names and shapes are the ten keys of the
problem statement's parameter table (tensortonic "Spatial Self-Attention",
parameter table):

* x ~ N(x_mean, x_std) of shape (B, C, H, W) (x_mean 0 for every workload)
* norm_weight = 1 + N(0, 0.1), norm_bias ~ N(0, 0.1), both (C,)
* q/k/v/out_weight ~ U(-1/sqrt(C), 1/sqrt(C)), (C, C)   (nn.Linear's range)
* q/k/v/out_bias ~ N(0, 0.02), (C,)

Draws are fp64 from ``numpy.random.default_rng(seed)`` in the fixed order
x, norm_weight, norm_bias, q_weight, q_bias, k_weight, k_bias, v_weight,
v_bias, out_weight, out_bias, then rounded once to the workload dtype.  The
rounded tensors are the inputs; the oracle upcasts them losslessly to fp64.

``stress=True`` draws the same numbers and then scales q_weight and k_weight
by 4 (peaked attention, score std near 5) and x by 0.05 (small residual), so
that an attention error cannot hide under the output's rounding.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

PARAM_KEYS = (
    "norm_weight", "norm_bias",
    "q_weight", "k_weight", "v_weight", "out_weight",
    "q_bias", "k_bias", "v_bias", "out_bias",
)

# Draw order (distinct from the ABI's parameter order): each weight with its bias.
_DRAW_ORDER = (
    "norm_weight", "norm_bias",
    "q_weight", "q_bias", "k_weight", "k_bias",
    "v_weight", "v_bias", "out_weight", "out_bias",
)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    C: int
    H: int
    W: int
    num_groups: int
    num_heads: int
    x_std: float = 1.0
    x_mean: float = 0.0  # a constant offset of every x value (a DC component)

    @property
    def T(self) -> int:
        return self.H * self.W

    @property
    def d(self) -> int:
        return self.C // self.num_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.dtype]

    def flops(self) -> int:
        """Algorithmic flops of one block: QKV 6BTC^2, QK^T and PV 4BT^2C, out-proj 2BTC^2."""
        B, T, C = self.B, self.T, self.C
        return 8 * B * T * C * C + 4 * B * T * T * C

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five measured workloads, indexed 0..4.
WORKLOADS = (
    Workload("fp32 B1 C64 8x8 G8 n2", "f32", 1, 64, 8, 8, 8, 2),
    Workload("BoTNet-c5 B64 C512 14x14 G32 n4", "bf16", 64, 512, 14, 14, 32, 4),
    Workload("DDPM mid-block B16 C512 16x16 G32 n8", "bf16", 16, 512, 16, 16, 32, 8),
    Workload("LDM level-1 B4 C320 64x64 G32 n5", "bf16", 4, 320, 64, 64, 32, 5),
    Workload("high-res B2 C640 96x96 G32 n10", "bf16", 2, 640, 96, 96, 32, 10, x_std=2.0),
)


def default_seed(index: int) -> int:
    return 1000 + index


def draw(wl: Workload, seed: int, stress: bool = False):
    """Return (x, params) as CPU torch tensors in the workload dtype.

    params is a dict keyed by PARAM_KEYS.
    """
    rng = np.random.default_rng(seed)
    B, C, H, W = wl.B, wl.C, wl.H, wl.W
    x = rng.standard_normal((B, C, H, W)) * wl.x_std + wl.x_mean
    bound = 1.0 / np.sqrt(C)
    raw = {}
    for key in _DRAW_ORDER:
        if key == "norm_weight":
            raw[key] = 1.0 + 0.1 * rng.standard_normal(C)
        elif key == "norm_bias":
            raw[key] = 0.1 * rng.standard_normal(C)
        elif key.endswith("_weight"):
            raw[key] = rng.uniform(-bound, bound, size=(C, C))
        else:
            raw[key] = 0.02 * rng.standard_normal(C)
    if stress:
        raw["q_weight"] = raw["q_weight"] * 4.0
        raw["k_weight"] = raw["k_weight"] * 4.0
        x = x * 0.05
    dt = wl.torch_dtype
    xt = torch.from_numpy(x).to(dt).contiguous()
    params = {k: torch.from_numpy(raw[k]).to(dt).contiguous() for k in PARAM_KEYS}
    return xt, params


def to_f64(x: torch.Tensor, params: dict):
    """Lossless upcast of the drawn tensors to fp64 numpy arrays (for the oracle).

    A None parameter (a projection without a bias) stays None."""
    return (x.to(torch.float64).numpy(),
            {k: (None if v is None else v.to(torch.float64).numpy()) for k, v in params.items()})


def draw_options(wl: Workload, seed: int, rel_pos: bool = False, qk_norm: bool = False,
                 rope: bool = False, stress: bool = False) -> dict:
    """Tensors of the optional steps, as CPU torch tensors in the workload dtype.

    rel_pos_table ((2H-1)(2W-1), n) ~ N(0, 1): logit shifts of order one, so
    the bias moves the attention visibly.  q/k norm gammas (n, d) ~
    U(0.5, 1.5) / sqrt(d) around the 1/sqrt(d) the qk-norm page starts from
    (normalised scores of order one); stress multiplies them by 3 (peaked
    attention).  Keys: rel_pos_table, q_norm_gamma, k_norm_gamma, rope; absent
    steps are None / False.
    """
    rng = np.random.default_rng(seed + 7919)
    H, W, n, d = wl.H, wl.W, wl.num_heads, wl.d
    dt = wl.torch_dtype
    out = {"rel_pos_table": None, "q_norm_gamma": None, "k_norm_gamma": None, "rope": rope}
    if rel_pos:
        t = rng.standard_normal(((2 * H - 1) * (2 * W - 1), n))
        out["rel_pos_table"] = torch.from_numpy(t).to(dt).contiguous()
    if qk_norm:
        g = 3.0 if stress else 1.0
        for k in ("q_norm_gamma", "k_norm_gamma"):
            v = g * rng.uniform(0.5, 1.5, size=(n, d)) / np.sqrt(d)
            out[k] = torch.from_numpy(v).to(dt).contiguous()
    return out


def options_f64(opts: dict) -> dict:
    """The oracle's keyword arguments for draw_options' tensors (fp64, lossless)."""
    f = lambda t: None if t is None else t.to(torch.float64).numpy()
    return {"rel_pos_table": f(opts["rel_pos_table"]), "q_norm_gamma": f(opts["q_norm_gamma"]),
            "k_norm_gamma": f(opts["k_norm_gamma"]), "rope_on": bool(opts["rope"])}


def draw_qkv(B: int, n: int, T: int, d: int, seed: int, kind: str = "peaked"):
    """Seeded per-head query, key and value tensors (B, n, T, d), bf16, for
    tests of the attention stage alone (written straight into the workspace).

    The query tensor is the one the attention stage reads: scores are
    2^(q . k), i.e. q already carries the score scale.
    * "peaked": q, k ~ N(0, 0.9) (score std near 6 in log2 units), v ~ N(0, 1);
    * "ramp": q ~ N(1, 0.2) and k ~ N(0, 0.2) + 4 t / T for key t, so scores
      grow along the key axis (the running maximum rises in every key block
      and early keys' weights underflow), v ~ N(0, 1).
    """
    rng = np.random.default_rng(seed)
    if kind == "peaked":
        q = 0.9 * rng.standard_normal((B, n, T, d))
        k = 0.9 * rng.standard_normal((B, n, T, d))
    elif kind == "ramp":
        q = 1.0 + 0.2 * rng.standard_normal((B, n, T, d))
        k = 0.2 * rng.standard_normal((B, n, T, d)) + (4.0 * np.arange(T) / T)[None, None, :, None]
    else:
        raise ValueError(kind)
    v = rng.standard_normal((B, n, T, d))
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16).contiguous()
    return to(q), to(k), to(v)
