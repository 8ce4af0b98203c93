"""Pins of the oracle's optional steps to facts fixed outside the oracle.

The steps come from the HNDL attention operator page (qkv_bias / out_bias
flags, rotary embeddings, 2-D relative-position bias) and vit-pytorch's
simple_vit_with_qk_norm.py (per-head query/key normalisation).  Sources of
truth used here, none of which is the oracle's own code:
* closed forms: a relative-position table that puts a huge logit on one
  offset makes every query copy the value row of the pixel at that offset,
  which fixes the sign, the axis and the stride of the index; rotary
  embedding at d = 2 is multiplication by e^{i t}; T = 1 leaves rotary
  embedding inert (stated on the page);
* invariants: softmax shift invariance (constant table), norm preservation and
  relative-position dependence of the rotation, scale invariance of the
  normalised queries and keys, the per-head norm sqrt(d) * gamma;
* an independent composition of torch fp64 routines (group_norm, linear,
  F.normalize, scaled_dot_product_attention with an additive mask) for all
  options together.
As in test_oracle_pins.py, a mutation test plants plausible mistakes in the
oracle's option code and checks that some pin catches each.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.ssa_oracle as ORA
from test_oracle_pins import rand_params, torch_gn


def maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))))


def draw(rng, B, C, H, W):
    return rng.standard_normal((B, C, H, W)), rand_params(rng, C)


# ---------------------------------------------------------------------------
# Nullable biases
# ---------------------------------------------------------------------------

def pin_bias_none_is_zero(ora):
    rng = np.random.default_rng(1)
    x, p = draw(rng, 2, 8, 3, 4)
    G, n = 2, 2
    for drop in (("q_bias", "k_bias", "v_bias"), ("out_bias",), ORA.BIAS_KEYS):
        pn = dict(p)
        pz = dict(p)
        for k in drop:
            pn[k] = None
            pz[k] = np.zeros(8)
        assert maxabs(ora.forward(x, pn, G, n), ora.forward(x, pz, G, n)) <= 1e-13


def pin_zero_out_weight_no_bias(ora):
    """Wo = 0 and no output bias: the attention branch vanishes, out = x exactly."""
    rng = np.random.default_rng(2)
    x, p = draw(rng, 2, 8, 3, 3)
    p["out_weight"] = np.zeros((8, 8))
    p["out_bias"] = None
    assert maxabs(ora.forward(x, p, 4, 2), x) == 0.0


# ---------------------------------------------------------------------------
# Relative-position bias
# ---------------------------------------------------------------------------

def value_rows(x, p, G):
    """V = GN(x) Wv^T + bv per pixel, from torch's group_norm (not the oracle)."""
    B, C, H, W = x.shape
    z = torch_gn(x, p, G).reshape(B, C, H * W).transpose(0, 2, 1)
    return z @ p["v_weight"].T + p["v_bias"]


def copy_neighbour(ora, dyo, dxo):
    """Table = +1e4 at the offset (dy, dx) = (row(q)-row(k), col(q)-col(k)) =
    (dyo, dxo), 0 elsewhere: every query whose neighbour at that offset exists
    takes that neighbour's value row exactly (softmax weight 1 - e^-1e4)."""
    rng = np.random.default_rng(3)
    B, C, H, W, G, n = 2, 8, 3, 4, 2, 2
    x, p = draw(rng, B, C, H, W)
    table = np.zeros(((2 * H - 1) * (2 * W - 1), n))
    table[(dyo + H - 1) * (2 * W - 1) + (dxo + W - 1), :] = 1e4
    out = ora.forward(x, p, G, n, rel_pos_table=table)
    V = value_rows(x, p, G)
    checked = 0
    for i in range(H):
        for j in range(W):
            ki, kj = i - dyo, j - dxo
            if not (0 <= ki < H and 0 <= kj < W):
                continue
            want = x[:, :, i, j] + V[:, ki * W + kj] @ p["out_weight"].T + p["out_bias"]
            assert maxabs(out[:, :, i, j], want) <= 1e-9
            checked += 1
    assert checked > 0


def pin_relpos_row_above(ora):
    copy_neighbour(ora, 1, 0)


def pin_relpos_column_left(ora):
    copy_neighbour(ora, 0, 1)


def pin_relpos_diagonal(ora):
    copy_neighbour(ora, -1, 2)


def pin_relpos_zero_and_constant_table(ora):
    """A zero table changes nothing; a constant table shifts whole score rows,
    which the softmax ignores -- so the bias enters the logits, before it."""
    rng = np.random.default_rng(4)
    x, p = draw(rng, 1, 8, 2, 3)
    L = 3 * 5
    base = ora.forward(x, p, 2, 2)
    assert maxabs(ora.forward(x, p, 2, 2, rel_pos_table=np.zeros((L, 2))), base) <= 1e-13
    assert maxabs(ora.forward(x, p, 2, 2, rel_pos_table=np.full((L, 2), 3.7)), base) <= 1e-12


# ---------------------------------------------------------------------------
# Rotary embeddings
# ---------------------------------------------------------------------------

def pin_rope_one_token_inert(ora):
    """At T == 1 the only angle is zero, so rope matches no rope (page statement)."""
    rng = np.random.default_rng(5)
    x, p = draw(rng, 3, 8, 1, 1)
    assert maxabs(ora.forward(x, p, 4, 2, rope_on=True), ora.forward(x, p, 4, 2)) <= 1e-13


def pin_rope_d2_is_complex_rotation(ora):
    """d = 2: theta_0 = 1, so the rotation multiplies a + ib by e^{i t}."""
    rng = np.random.default_rng(6)
    X = rng.standard_normal((1, 1, 7, 2))
    t = np.arange(7)
    z = (X[0, 0, :, 0] + 1j * X[0, 0, :, 1]) * np.exp(1j * t)
    R = ora.rope(X, t)
    assert maxabs(R[0, 0, :, 0], z.real) <= 1e-12 and maxabs(R[0, 0, :, 1], z.imag) <= 1e-12


def pin_rope_norm_and_relative(ora):
    """A rotation keeps norms, and q.k after rotation depends on the positions
    only through their difference (to float32 angle rounding)."""
    rng = np.random.default_rng(7)
    d = 16
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 1, d))
    assert abs(np.linalg.norm(ora.rope(q, [37])) - np.linalg.norm(q)) <= 1e-12
    dots = []
    for shift in (0, 5, 29):
        dots.append(float((ora.rope(q, [11 + shift]) * ora.rope(k, [4 + shift])).sum()))
    assert max(dots) - min(dots) <= 1e-4 * np.linalg.norm(q) * np.linalg.norm(k)
    # and it does depend on the difference
    other = float((ora.rope(q, [11]) * ora.rope(k, [6])).sum())
    assert abs(other - dots[0]) > 1e-3


# ---------------------------------------------------------------------------
# Query/key normalisation
# ---------------------------------------------------------------------------

def pin_qknorm_scale_invariance(ora):
    """Normalised queries and keys forget the projections' scale."""
    rng = np.random.default_rng(8)
    x, p = draw(rng, 2, 8, 3, 3)
    gq, gk = rng.uniform(0.5, 1.5, (2, 4)), rng.uniform(0.5, 1.5, (2, 4))
    base = ora.forward(x, p, 2, 2, q_norm_gamma=gq, k_norm_gamma=gk)
    ps = dict(p)
    ps["q_weight"], ps["q_bias"] = 3.0 * p["q_weight"], 3.0 * p["q_bias"]
    ps["k_weight"], ps["k_bias"] = 0.25 * p["k_weight"], 0.25 * p["k_bias"]
    assert maxabs(ora.forward(x, ps, 2, 2, q_norm_gamma=gq, k_norm_gamma=gk), base) <= 1e-12
    # without the normalisation the same rescale does change the output
    assert maxabs(ora.forward(x, ps, 2, 2), ora.forward(x, p, 2, 2)) > 1e-6


def pin_qknorm_head_norms(ora):
    """With gamma = c everywhere each head's query has norm sqrt(d) * c."""
    rng = np.random.default_rng(9)
    x, p = draw(rng, 1, 12, 2, 3)
    n, d, c = 3, 4, 0.7
    g = np.full((n, d), c)
    st = ora.forward_stages(x, p, 3, n, q_norm_gamma=g, k_norm_gamma=g)
    Qh = st["Q"].reshape(1, 6, n, d)
    assert maxabs(np.linalg.norm(Qh, axis=-1), math.sqrt(d) * c) <= 1e-12


# ---------------------------------------------------------------------------
# All options together: torch fp64 composition
# ---------------------------------------------------------------------------

def torch_block_options(x, p, G, n, table, gq, gk, rope_on):
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float64))
    xt = t(x)
    B, C, H, W = xt.shape
    T, d = H * W, C // n
    gn = F.group_norm(xt, G, t(p["norm_weight"]), t(p["norm_bias"]), eps=1e-5)
    z = gn.flatten(2).transpose(1, 2)
    heads = lambda m: m.view(B, T, n, d).transpose(1, 2)
    q = heads(F.linear(z, t(p["q_weight"]), t(p["q_bias"])))
    k = heads(F.linear(z, t(p["k_weight"]), t(p["k_bias"])))
    v = heads(F.linear(z, t(p["v_weight"]), t(p["v_bias"])))
    scale = 1.0 / math.sqrt(d)
    if gq is not None:
        q = F.normalize(q, dim=-1) * math.sqrt(d) * t(gq)[None, :, None, :]
        k = F.normalize(k, dim=-1) * math.sqrt(d) * t(gk)[None, :, None, :]
        scale = 1.0
    if rope_on:
        i = torch.arange(d // 2, dtype=torch.float32)
        theta = torch.pow(torch.tensor(10000.0, dtype=torch.float64), -2.0 * i.double() / d).float()
        ang = (torch.arange(T, dtype=torch.float32)[:, None] * theta[None, :]).double()
        cos, sin = torch.cos(ang).repeat(1, 2), torch.sin(ang).repeat(1, 2)
        rot = lambda m: torch.cat([-m[..., d // 2:], m[..., : d // 2]], dim=-1)
        q, k = q * cos + rot(q) * sin, k * cos + rot(k) * sin
    mask = None
    if table is not None:
        yy, xx = torch.meshgrid(torch.arange(H), torch.arange(W), indexing="ij")
        r, c = yy.flatten(), xx.flatten()
        idx = (r[:, None] - r[None, :] + H - 1) * (2 * W - 1) + (c[:, None] - c[None, :] + W - 1)
        mask = t(table)[idx].permute(2, 0, 1)[None]     # (1, n, T, T)
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    y = F.linear(o.transpose(1, 2).reshape(B, T, C), t(p["out_weight"]), t(p["out_bias"]))
    return (xt + y.transpose(1, 2).reshape(B, C, H, W)).numpy()


def pin_torch_all_options(ora):
    rng = np.random.default_rng(10)
    for (B, C, H, W, G, n) in ((2, 8, 3, 4, 2, 2), (1, 12, 2, 5, 3, 3), (1, 16, 4, 4, 4, 2)):
        x, p = draw(rng, B, C, H, W)
        d = C // n
        table = rng.standard_normal(((2 * H - 1) * (2 * W - 1), n))
        gq, gk = rng.uniform(0.5, 1.5, (n, d)), rng.uniform(0.5, 1.5, (n, d))
        p["k_bias"] = None
        for opts in ({"rel_pos_table": table}, {"rope_on": True},
                     {"q_norm_gamma": gq, "k_norm_gamma": gk},
                     {"rel_pos_table": table, "rope_on": True, "q_norm_gamma": gq, "k_norm_gamma": gk}):
            want = torch_block_options(x, p, G, n, opts.get("rel_pos_table"), opts.get("q_norm_gamma"),
                                       opts.get("k_norm_gamma"), opts.get("rope_on", False))
            assert maxabs(ora.forward(x, p, G, n, **opts), want) <= 1e-10


def pin_forward_pixels_options(ora):
    rng = np.random.default_rng(11)
    x, p = draw(rng, 2, 8, 3, 5)
    n, d = 2, 4
    opts = {"rel_pos_table": rng.standard_normal((5 * 9, n)), "rope_on": True,
            "q_norm_gamma": rng.uniform(0.5, 1.5, (n, d)), "k_norm_gamma": rng.uniform(0.5, 1.5, (n, d))}
    full = ora.forward(x, p, 2, n, **opts)
    rows = [0, 4, 7, 14]
    got = ora.forward_pixels(x, p, 2, n, 1, rows, **opts)
    assert maxabs(got, full[1].reshape(8, 15)[:, rows]) <= 1e-12


PINS = [
    pin_bias_none_is_zero, pin_zero_out_weight_no_bias,
    pin_relpos_row_above, pin_relpos_column_left, pin_relpos_diagonal,
    pin_relpos_zero_and_constant_table,
    pin_rope_one_token_inert, pin_rope_d2_is_complex_rotation, pin_rope_norm_and_relative,
    pin_qknorm_scale_invariance, pin_qknorm_head_norms,
    pin_torch_all_options, pin_forward_pixels_options,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ORA)


def test_check_options_rejects():
    with pytest.raises(ValueError):
        ORA.check_options(8, 3, 4, 2, np.zeros((10, 2)), None, None, False)
    with pytest.raises(ValueError):
        ORA.check_options(8, 3, 4, 2, None, np.ones((2, 4)), None, False)
    with pytest.raises(ValueError):
        ORA.check_options(6, 3, 4, 2, None, None, None, True)   # d = 3 is odd


# ---------------------------------------------------------------------------
# Mutation test: plausible mistakes in the option code must be caught
# ---------------------------------------------------------------------------

_ORIG_REL = ORA.rel_pos_bias
_ORIG_ROPE = ORA.rope
_ORIG_QKN = ORA.qk_norm
_ORIG_STAGES = ORA.forward_stages


def _rel_variant(kind):
    def f(table, H, W, rows=None):
        table = np.asarray(table, dtype=np.float64)
        T = H * W
        q = np.arange(T) if rows is None else np.asarray(rows)
        k = np.arange(T)
        sgn = -1 if kind == "sign" else 1
        dy = sgn * ((q // W)[:, None] - (k // W)[None, :]) + (H - 1)
        dx = sgn * ((q % W)[:, None] - (k % W)[None, :]) + (W - 1)
        if kind == "stride":
            idx = dy * (2 * H - 1) + dx
        elif kind == "swap":
            idx = dx * (2 * H - 1) + dy
        else:
            idx = dy * (2 * W - 1) + dx
        idx = np.clip(idx, 0, table.shape[0] - 1)
        return table[idx].transpose(2, 0, 1)
    return f


def _rope_variant(kind):
    def f(Xh, positions):
        Xh = np.asarray(Xh, dtype=np.float64)
        d = Xh.shape[-1]
        ang = ORA.rope_angles(positions, d)
        if kind == "interleaved":   # pairs (2i, 2i+1) instead of halves
            a, b = Xh[..., 0::2], Xh[..., 1::2]
            out = np.empty_like(Xh)
            out[..., 0::2] = a * np.cos(ang) - b * np.sin(ang)
            out[..., 1::2] = b * np.cos(ang) + a * np.sin(ang)
            return out
        cos = np.concatenate([np.cos(ang)] * 2, axis=-1)
        sin = np.concatenate([np.sin(ang)] * 2, axis=-1)
        a, b = Xh[..., : d // 2], Xh[..., d // 2:]
        rot = np.concatenate([b, -a], axis=-1)          # "sign": rotate the other way
        return Xh * cos + rot * sin
    return f


def _qkn_token_axis(Xh, gamma):
    Xh = np.asarray(Xh, dtype=np.float64)
    d = Xh.shape[-1]
    nrm = np.sqrt((Xh * Xh).sum(axis=-2, keepdims=True))
    return Xh / np.maximum(nrm, 1e-12) * np.sqrt(d) * np.asarray(gamma)[None, :, None, :]


def _qkn_no_gamma(Xh, gamma):
    return _ORIG_QKN(Xh, np.full(np.shape(gamma), 1.0 / math.sqrt(np.shape(gamma)[1])))


def _stages_keep_scale(x, params, G, n, **opts):
    """QK-norm that still divides the scores by sqrt(d)."""
    if opts.get("q_norm_gamma") is None:
        return _ORIG_STAGES(x, params, G, n, **opts)
    s = 1.0 / math.sqrt(params["q_weight"].shape[0] // n) ** 0.5
    o = dict(opts)
    o["q_norm_gamma"] = np.asarray(opts["q_norm_gamma"]) * s
    o["k_norm_gamma"] = np.asarray(opts["k_norm_gamma"]) * s
    return _ORIG_STAGES(x, params, G, n, **o)


def _stages_bias_after_softmax(x, params, G, n, **opts):
    table = opts.get("rel_pos_table")
    if table is None:
        return _ORIG_STAGES(x, params, G, n, **opts)
    o = dict(opts)
    o["rel_pos_table"] = None
    st = _ORIG_STAGES(x, params, G, n, **o)
    B, C, H, W = np.shape(x)
    bias = ORA.rel_pos_bias(table, H, W)
    Vh = ORA.split_heads(st["V"], n)
    Oh = (st["P"] + bias[None] * 1e-3) @ Vh
    Y = ORA.linear(ORA.merge_heads(Oh), params["out_weight"], params["out_bias"])
    st["out"] = np.asarray(x, dtype=np.float64) + ORA.image(Y, H, W)
    return st


def _linear_bias_none_as_one(z, weight, bias):
    y = np.asarray(z, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T
    return y + (1.0 if bias is None else np.asarray(bias, dtype=np.float64))


MUTANTS = {
    "relpos dy/dx sign": ("rel_pos_bias", _rel_variant("sign")),
    "relpos stride 2H-1": ("rel_pos_bias", _rel_variant("stride")),
    "relpos rows and cols swapped": ("rel_pos_bias", _rel_variant("swap")),
    "relpos after softmax": ("forward_stages", _stages_bias_after_softmax),
    "rope interleaved pairs": ("rope", _rope_variant("interleaved")),
    "rope opposite rotation": ("rope", _rope_variant("sign")),
    "qknorm over tokens": ("qk_norm", _qkn_token_axis),
    "qknorm drops gamma": ("qk_norm", _qkn_no_gamma),
    "qknorm keeps 1/sqrt(d)": ("forward_stages", _stages_keep_scale),
    "missing bias read as one": ("linear", _linear_bias_none_as_one),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ORA, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(ORA)
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"
