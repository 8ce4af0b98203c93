"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Sources of truth used here, none of which is the oracle's own code:
* the worked examples printed on the tensortonic "Spatial Self-Attention"
  problem page (tests/golden/page1_examples.json);
* closed forms the block reduces to (one pixel, zero weights, uniform
  attention, two tokens);
* invariants (k_bias invariance, v_bias shift, pixel-permutation
  equivariance, GroupNorm moments, softmax rows);
* an independent composition of torch's fp64 library routines
  (group_norm, linear, scaled_dot_product_attention);
* a scalar brute force in plain Python at the worked examples' shapes.

Every pin is a function of the oracle module, so the mutation test at the
bottom can plant a mistake in the oracle and check that some pin catches it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.ssa_oracle as ORA

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "page1_examples.json")))["examples"]
KEYS = ORA.PARAM_KEYS


def rand_params(rng, C, wscale=1.0):
    """Random fp64 parameters with non-symmetric weights and non-zero biases."""
    p = {
        "norm_weight": 1.0 + 0.3 * rng.standard_normal(C),
        "norm_bias": 0.3 * rng.standard_normal(C),
    }
    for k in ("q", "k", "v", "out"):
        p[f"{k}_weight"] = wscale * rng.standard_normal((C, C)) / math.sqrt(C)
        p[f"{k}_bias"] = 0.2 * rng.standard_normal(C)
    return p


def torch_block(x, p, G, n):
    """The block composed from torch fp64 library routines (independent of the oracle)."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    xt = t(x)
    B, C, H, W = xt.shape
    T, d = H * W, C // n
    gn = F.group_norm(xt, G, t(p["norm_weight"]), t(p["norm_bias"]), eps=1e-5)
    z = gn.flatten(2).transpose(1, 2)
    q = F.linear(z, t(p["q_weight"]), t(p["q_bias"])).view(B, T, n, d).transpose(1, 2)
    k = F.linear(z, t(p["k_weight"]), t(p["k_bias"])).view(B, T, n, d).transpose(1, 2)
    v = F.linear(z, t(p["v_weight"]), t(p["v_bias"])).view(B, T, n, d).transpose(1, 2)
    o = F.scaled_dot_product_attention(q, k, v)       # default scale 1/sqrt(d)
    o = o.transpose(1, 2).reshape(B, T, C)
    y = F.linear(o, t(p["out_weight"]), t(p["out_bias"]))
    return (xt + y.transpose(1, 2).reshape(B, C, H, W)).numpy()


def torch_gn(x, p, G):
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    return F.group_norm(t(x), G, t(p["norm_weight"]), t(p["norm_bias"]), eps=1e-5).numpy()


def brute_force(x, p, G, n):
    """Scalar loops over the page's definition, in plain Python floats."""
    B, C, H, W = x.shape
    T, d, Cg = H * W, C // n, C // G
    out = np.array(x, dtype=np.float64)
    for b in range(B):
        z = [[0.0] * C for _ in range(T)]
        for g in range(G):
            vals = [float(x[b, c, i, j]) for c in range(g * Cg, (g + 1) * Cg)
                    for i in range(H) for j in range(W)]
            mu = sum(vals) / len(vals)
            var = sum((v - mu) ** 2 for v in vals) / len(vals)
            for c in range(g * Cg, (g + 1) * Cg):
                for i in range(H):
                    for j in range(W):
                        xh = (float(x[b, c, i, j]) - mu) / math.sqrt(var + 1e-5)
                        z[i * W + j][c] = xh * p["norm_weight"][c] + p["norm_bias"][c]

        def lin(rows, Wm, bv):
            return [[sum(r[c] * Wm[o][c] for c in range(C)) + bv[o] for o in range(C)] for r in rows]

        q = lin(z, p["q_weight"], p["q_bias"])
        k = lin(z, p["k_weight"], p["k_bias"])
        v = lin(z, p["v_weight"], p["v_bias"])
        o = [[0.0] * C for _ in range(T)]
        for h in range(n):
            ch = range(h * d, (h + 1) * d)
            for t in range(T):
                s = [sum(q[t][c] * k[u][c] for c in ch) / math.sqrt(d) for u in range(T)]
                m = max(s)
                e = [math.exp(si - m) for si in s]
                tot = sum(e)
                for c in ch:
                    o[t][c] = sum(e[u] / tot * v[u][c] for u in range(T))
        y = lin(o, p["out_weight"], p["out_bias"])
        for c in range(C):
            for i in range(H):
                for j in range(W):
                    out[b, c, i, j] = float(x[b, c, i, j]) + y[i * W + j][c]
    return out


def maxabs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))))


# ---------------------------------------------------------------------------
# Pins.  Each takes the oracle module and asserts.
# ---------------------------------------------------------------------------

def pin_example3_structure(ora):
    """Third worked example: one pixel, one channel per group.

    Each group then holds a single value, so GN(x) is exactly norm_bias and
    out - x = (norm_bias Wv^T + bv) Wo^T + bo for every sample, whatever x is.
    """
    ex = GOLDEN[2]
    x = np.array(ex["x"])
    rng = np.random.default_rng(3)
    p = rand_params(rng, 4)
    out = ora.forward(x, p, ex["num_groups"], ex["num_heads"])
    delta = out - x
    want = (p["norm_bias"] @ p["v_weight"].T + p["v_bias"]) @ p["out_weight"].T + p["out_bias"]
    assert maxabs(delta[0, :, 0, 0], want) < 1e-12
    assert maxabs(delta[1, :, 0, 0], want) < 1e-12
    x2 = x + rng.standard_normal(x.shape)
    assert maxabs(ora.forward(x2, p, 4, 2) - x2, delta) < 1e-12


def pin_hw1_closed_form(ora):
    """One pixel with several channels per group: a single key gets weight 1,
    so out = x + (GN(x) Wv^T + bv) Wo^T + bo, with GN taken from torch."""
    rng = np.random.default_rng(4)
    B, C, G, n = 3, 8, 2, 4
    x = rng.standard_normal((B, C, 1, 1)) * 1.7 + 0.3
    p = rand_params(rng, C)
    gn = torch_gn(x, p, G)[:, :, 0, 0]
    want = x[:, :, 0, 0] + (gn @ p["v_weight"].T + p["v_bias"]) @ p["out_weight"].T + p["out_bias"]
    assert maxabs(ora.forward(x, p, G, n)[:, :, 0, 0], want) < 1e-12


def pin_zero_weights(ora):
    """Zero projection weights give out = x + bo; Wo = 0 alone does too."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 6, 2, 3))
    p = rand_params(rng, 6)
    for k in ("q_weight", "k_weight", "v_weight", "out_weight"):
        p[k] = np.zeros((6, 6))
    want = x + p["out_bias"][None, :, None, None]
    assert maxabs(ora.forward(x, p, 3, 2), want) < 1e-12
    p2 = rand_params(rng, 6)
    p2["out_weight"] = np.zeros((6, 6))
    want2 = x + p2["out_bias"][None, :, None, None]
    assert maxabs(ora.forward(x, p2, 2, 3), want2) < 1e-12


def pin_uniform_attention(ora):
    """Wq = 0 and bq = 0 make every score 0, so each query averages all pixels:
    out = x + ((mean_t Z) Wv^T + bv) Wo^T + bo at every pixel, Z from torch's GN."""
    rng = np.random.default_rng(6)
    B, C, H, W, G, n = 2, 8, 3, 4, 4, 2
    x = rng.standard_normal((B, C, H, W))
    p = rand_params(rng, C)
    p["q_weight"] = np.zeros((C, C))
    p["q_bias"] = np.zeros(C)
    zbar = torch_gn(x, p, G).mean(axis=(2, 3))                        # (B, C)
    y = (zbar @ p["v_weight"].T + p["v_bias"]) @ p["out_weight"].T + p["out_bias"]
    want = x + y[:, :, None, None]
    assert maxabs(ora.forward(x, p, G, n), want) < 1e-12


def pin_two_token_logistic(ora):
    """Two pixels, one head: softmax over two keys is the logistic function of
    the score difference, which fixes the 1/sqrt(d) scale and the key axis."""
    rng = np.random.default_rng(7)
    B, C, H, W, G, n = 2, 6, 1, 2, 3, 1
    x = rng.standard_normal((B, C, H, W))
    p = rand_params(rng, C, wscale=2.0)
    z = torch_gn(x, p, G).reshape(B, C, 2).transpose(0, 2, 1)        # (B, 2, C)
    q = z @ p["q_weight"].T + p["q_bias"]
    k = z @ p["k_weight"].T + p["k_bias"]
    v = z @ p["v_weight"].T + p["v_bias"]
    want = np.empty_like(x)
    for b in range(B):
        for t in range(2):
            dlt = (q[b, t] @ k[b, 0] - q[b, t] @ k[b, 1]) / math.sqrt(C)
            w0 = 1.0 / (1.0 + math.exp(-dlt))
            o = w0 * v[b, 0] + (1.0 - w0) * v[b, 1]
            want[b, :, 0, t] = x[b, :, 0, t] + o @ p["out_weight"].T + p["out_bias"]
    assert maxabs(ora.forward(x, p, G, n), want) < 1e-12


def pin_bv_shift(ora):
    """Rows of P sum to one, so bv -> bv + delta shifts every pixel by delta Wo^T."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 8, 3, 3))
    p = rand_params(rng, 8, wscale=2.0)
    delta = rng.standard_normal(8)
    p2 = dict(p, v_bias=p["v_bias"] + delta)
    shift = delta @ p["out_weight"].T
    got = ora.forward(x, p2, 4, 4) - ora.forward(x, p, 4, 4)
    assert maxabs(got, np.broadcast_to(shift[None, :, None, None], got.shape)) < 1e-12


def pin_k_bias_invariance(ora):
    """bk adds q_t . bk_j / sqrt(d) to a whole score row; softmax ignores that."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 8, 2, 3))
    p = rand_params(rng, 8, wscale=2.0)
    p2 = dict(p, k_bias=3.0 * rng.standard_normal(8))
    assert maxabs(ora.forward(x, p, 2, 2), ora.forward(x, p2, 2, 2)) < 1e-12


def pin_permutation_equivariance(ora):
    """No positional term: permuting the pixels permutes the output the same way."""
    rng = np.random.default_rng(10)
    for (H, W) in ((2, 3), (4, 4)):
        x = rng.standard_normal((2, 8, H, W))
        p = rand_params(rng, 8, wscale=2.0)
        perm = rng.permutation(H * W)
        xp = x.reshape(2, 8, H * W)[:, :, perm].reshape(x.shape)
        a = ora.forward(x, p, 4, 2).reshape(2, 8, H * W)[:, :, perm]
        b = ora.forward(xp, p, 4, 2).reshape(2, 8, H * W)
        assert maxabs(a, b) < 1e-12


def pin_torch_composition_small(ora):
    """Independent fp64 composition of torch routines at small shapes, incl. the page's."""
    rng = np.random.default_rng(11)
    shapes = [(1, 4, 2, 2, 2, 2), (1, 2, 2, 3, 1, 1), (2, 4, 1, 1, 4, 2),
              (2, 12, 3, 5, 3, 3), (1, 64, 8, 8, 8, 2)]
    for (B, C, H, W, G, n) in shapes:
        x = rng.standard_normal((B, C, H, W)) * 1.5
        p = rand_params(rng, C, wscale=2.0)
        assert maxabs(ora.forward(x, p, G, n), torch_block(x, p, G, n)) < 1e-10


def pin_brute_force(ora):
    """Scalar-loop evaluation at the three worked examples' shapes."""
    rng = np.random.default_rng(12)
    for ex in GOLDEN:
        x = np.array(ex["x"])
        C = x.shape[1]
        p = rand_params(rng, C, wscale=2.0)
        got = ora.forward(x, p, ex["num_groups"], ex["num_heads"])
        assert maxabs(got, brute_force(x, p, ex["num_groups"], ex["num_heads"])) < 1e-12


def pin_gn_moments(ora):
    """Per group the normalised values have mean 0 and mean square var/(var+eps),
    and the statistics match the plain two-pass definition on a constant group."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 12, 4, 5)) * 0.01 + 2.0
    ones, zeros = np.ones(12), np.zeros(12)
    xh, mean, var = ora.group_norm(x, ones, zeros, 3)
    xg = xh.reshape(3, 3, -1)
    assert np.max(np.abs(xg.mean(axis=2))) < 1e-9
    assert np.max(np.abs((xg ** 2).mean(axis=2) - var / (var + 1e-5))) < 1e-9
    c = np.full((1, 4, 2, 2), 7.0)
    xh2, m2, v2 = ora.group_norm(c, np.ones(4), np.zeros(4), 2)
    assert np.all(m2 == 7.0) and np.all(v2 == 0.0) and np.all(xh2 == 0.0)


def pin_softmax_rows(ora):
    """Rows are non-negative, sum to one, and ignore a constant shift."""
    rng = np.random.default_rng(14)
    S = rng.standard_normal((3, 5, 7)) * 4
    P = ora.softmax_keys(S)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(axis=-1) - 1)) < 1e-14
    assert maxabs(ora.softmax_keys(S + 123.0), P) < 1e-14
    big = ora.softmax_keys(np.array([[1000.0, 0.0, -1000.0]]))
    assert maxabs(big, [[1.0, 0.0, 0.0]]) < 1e-300 + 1e-15


def pin_tokens_order(ora):
    """Pixel (i, j) becomes token row i*W + j, and image() undoes tokens()."""
    rng = np.random.default_rng(15)
    img = rng.standard_normal((2, 3, 4, 5))
    tok = ora.tokens(img)
    for b in range(2):
        for c in range(3):
            for i in range(4):
                for j in range(5):
                    assert tok[b, i * 5 + j, c] == img[b, c, i, j]
    assert np.array_equal(ora.image(tok, 4, 5), img)


def pin_forward_pixels(ora):
    """The sampled-pixel evaluation equals the full forward at those pixels."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((3, 12, 5, 7))
    p = rand_params(rng, 12, wscale=2.0)
    full = ora.forward(x, p, 4, 3).reshape(3, 12, 35)
    rows = [0, 6, 17, 34]
    assert maxabs(ora.forward_pixels(x, p, 4, 3, 1, rows), full[1][:, rows]) < 1e-12


PINS = [
    pin_example3_structure, pin_hw1_closed_form, pin_zero_weights,
    pin_uniform_attention, pin_two_token_logistic, pin_bv_shift,
    pin_k_bias_invariance, pin_permutation_equivariance,
    pin_torch_composition_small, pin_brute_force, pin_gn_moments,
    pin_softmax_rows, pin_tokens_order, pin_forward_pixels,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ORA)


# ---------------------------------------------------------------------------
# Facts about the page's own printed data.
# ---------------------------------------------------------------------------

def test_page_example3_residual_is_sample_independent():
    """The printed third example has out - x equal across its two samples (to
    print rounding), as the one-pixel reading of GN + residual requires."""
    ex = GOLDEN[2]
    x, out = np.array(ex["x"]), np.array(ex["out"])
    delta = out - x
    assert maxabs(delta[0], delta[1]) <= 2e-6
    assert maxabs(delta[0, :, 0, 0], [-0.118129, -0.165209, -0.143070, 0.171774]) <= 1e-6


def test_page_example1_attention_row_is_a_distribution():
    """The printed attention row of the first example is non-negative and sums
    to one within its three-decimal rounding."""
    row = np.array(GOLDEN[0]["attention_row_head0_pixel0"])
    assert np.all(row > 0)
    assert abs(row.sum() - 1.0) <= 4 * 0.0005


def test_example_output_shapes():
    rng = np.random.default_rng(17)
    for ex in GOLDEN:
        x = np.array(ex["x"])
        p = rand_params(rng, x.shape[1])
        assert ORA.forward(x, p, ex["num_groups"], ex["num_heads"]).shape == np.array(ex["out"]).shape


def test_check_args_rejects():
    rng = np.random.default_rng(18)
    x = rng.standard_normal((1, 6, 2, 2))
    p = rand_params(rng, 6)
    with pytest.raises(ValueError):
        ORA.forward(x, p, 4, 2)          # 4 does not divide 6
    with pytest.raises(ValueError):
        ORA.forward(x, p, 3, 4)          # 4 does not divide 6
    bad = dict(p, q_weight=np.zeros((6, 5)))
    with pytest.raises(ValueError):
        ORA.forward(x, bad, 3, 2)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_torch_composition_workload_channels(idx):
    """The torch composition again, at each measured workload's channel, group
    and head counts (batch cut to one sample, spatial size cut to keep the
    CPU suite short)."""
    from spatial_self_attention_amd.inputs import WORKLOADS, draw, to_f64
    wl = WORKLOADS[idx]
    side = {1: 14, 2: 16, 3: 24, 4: 12}[idx]
    wl = wl.replace(B=1, H=side, W=side, dtype="f32")
    x, p = to_f64(*draw(wl, 2000 + idx))
    got = ORA.forward(x, p, wl.num_groups, wl.num_heads)
    assert maxabs(got, torch_block(x, p, wl.num_groups, wl.num_heads)) < 1e-10


# ---------------------------------------------------------------------------
# Mutation test: plant plausible mistakes in the oracle and make sure at least
# one pin fails for each.
# ---------------------------------------------------------------------------

def _mut_linear_no_transpose(z, weight, bias):
    return np.asarray(z) @ np.asarray(weight) + bias


def _mut_linear_no_bias(z, weight, bias):
    return np.asarray(z) @ np.asarray(weight).T


def _mut_softmax_query_axis(S):
    S = np.asarray(S)
    e = np.exp(S - S.max(axis=-2, keepdims=True))
    return e / e.sum(axis=-2, keepdims=True)


def _mk_attention(scale_fn=None, reverse_heads=False):
    def att(Q, K, V, num_heads):
        B, T, C = Q.shape
        d = C // num_heads
        O = np.empty_like(Q)
        P = np.empty((B, num_heads, T, T))
        for j in range(num_heads):
            sl = slice(j * d, (j + 1) * d)
            dst = slice((num_heads - 1 - j) * d, (num_heads - j) * d) if reverse_heads else sl
            S = Q[:, :, sl] @ K[:, :, sl].transpose(0, 2, 1) / scale_fn(d)
            P[:, j] = ORA.softmax_keys(S)
            O[:, :, dst] = P[:, j] @ V[:, :, sl]
        return O, P
    return att


def _mk_group_norm(kind):
    def gn(x, weight, bias, num_groups, eps=1e-5):
        x = np.asarray(x, dtype=np.float64)
        B, C, H, W = x.shape
        G = num_groups
        if kind == "interleaved":
            xg = x.reshape(B, C // G, G, H * W).transpose(0, 2, 1, 3).reshape(B, G, -1)
        else:
            xg = x.reshape(B, G, -1)
        mean = xg.mean(axis=2)
        if kind == "unbiased":
            var = ((xg - mean[:, :, None]) ** 2).sum(axis=2) / (xg.shape[2] - 1 if xg.shape[2] > 1 else 1)
        else:
            var = ((xg - mean[:, :, None]) ** 2).mean(axis=2)
        if kind == "eps_outside":
            xh = (xg - mean[:, :, None]) / (np.sqrt(var[:, :, None]) + eps)
        else:
            xh = (xg - mean[:, :, None]) / np.sqrt(var[:, :, None] + eps)
        if kind == "interleaved":
            xh = xh.reshape(B, G, C // G, H * W).transpose(0, 2, 1, 3)
        xh = xh.reshape(B, C, H, W)
        return xh * weight[None, :, None, None] + bias[None, :, None, None], mean, var
    return gn


def _mut_image_transposed(tok, H, W):
    tok = np.asarray(tok)
    B, T, C = tok.shape
    return tok.transpose(0, 2, 1).reshape(B, C, W, H).transpose(0, 1, 3, 2)


_ORIG_FORWARD_STAGES = ORA.forward_stages


def _mut_forward_residual_gn(x, params, num_groups, num_heads):
    st = _ORIG_FORWARD_STAGES(x, params, num_groups, num_heads)
    gn, _, _ = ORA.group_norm(x, params["norm_weight"], params["norm_bias"], num_groups)
    st["out"] = st["out"] - np.asarray(x) + gn
    return st


MUTANTS = {
    "linear W not transposed": ("linear", _mut_linear_no_transpose),
    "linear bias dropped": ("linear", _mut_linear_no_bias),
    "softmax over queries": ("softmax_keys", _mut_softmax_query_axis),
    "scores divided by d": ("attention", _mk_attention(lambda d: d)),
    "scores not scaled": ("attention", _mk_attention(lambda d: 1.0)),
    "heads concatenated in reverse": ("attention", _mk_attention(math.sqrt, reverse_heads=True)),
    "GN eps outside sqrt": ("group_norm", _mk_group_norm("eps_outside")),
    "GN unbiased variance": ("group_norm", _mk_group_norm("unbiased")),
    "GN interleaved groups": ("group_norm", _mk_group_norm("interleaved")),
    "image transposes H and W": ("image", _mut_image_transposed),
    "residual adds GN(x)": ("forward_stages", _mut_forward_residual_gn),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ORA, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(ORA)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"
