"""fp64 CPU oracle of the spatial self-attention block.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the package's smoke
check and the benchmark's CPU-baseline leg may import this module.  It shares
no code with the HIP path and imports nothing from it.

What it computes is the block defined by the tensortonic problem "Spatial
Self-Attention" (diffusion-from-scratch study plan, L03), formula and the
prose under it:

    Z   = tokens(GN(x))
    Q   = Z Wq^T + bq,  K = Z Wk^T + bk,  V = Z Wv^T + bv
    O_j = softmax(Q_j K_j^T / sqrt(d)) V_j          for heads j = 0..n-1
    out = x + image([O_1, ..., O_n] Wo^T + bo)

written out plainly in float64 with NumPy.  Each helper names the passage it
follows.  Where the page is garbled or silent, the reading taken is stated at
the helper (the radical in the score scale, GroupNorm's grouping and variance,
the weight orientation).

Optional steps, from the other pages (each off by default, so the block above
is unchanged when none is given):
* a projection without a bias (the HNDL attention operator's qkv_bias /
  out_bias flags: "a projection built without a bias has no bias parameter");
* per-head query/key normalisation (vit-pytorch simple_vit_with_qk_norm.py,
  RMSNorm: x / ||x|| * sqrt(d) * gamma, and then no 1/sqrt(d) on the scores);
* rotary position embeddings over the token index (HNDL attention operator,
  "Rotary embeddings");
* a learned 2-D relative-position bias added to the scaled logits (HNDL
  attention operator, "Relative position bias").
Order of the steps: projections, query/key normalisation, rotary embedding,
scaled scores plus the position bias, softmax over keys, P V.

Pinned against the pages and the mathematics by tests/test_oracle_pins.py
(closed forms, invariants, an independent torch fp64 composition, scalar
brute force).  Only the printed output values of the page's first two worked
examples are parity unpinned (their parameters are not printed).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-5  # GroupNorm epsilon fixed by the problem statement's prose.

PARAM_KEYS = (
    "norm_weight", "norm_bias",
    "q_weight", "k_weight", "v_weight", "out_weight",
    "q_bias", "k_bias", "v_bias", "out_bias",
)


BIAS_KEYS = ("q_bias", "k_bias", "v_bias", "out_bias")


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def check_args(x, params, num_groups: int, num_heads: int):
    """Shape rules of the parameter table (tensortonic problem, parameter table).

    x is (B, C, H, W); norm_* and the biases are (C,); the four weights are
    (C, C).  The group count and head count must divide C (head j takes a
    contiguous block of d = C/n channels; the HNDL attention spec reports a
    constraint error when heads do not divide the width).
    """
    x = _f64(x)
    if x.ndim != 4:
        raise ValueError("x must be (B, C, H, W)")
    B, C, H, W = x.shape
    for k in PARAM_KEYS:
        if k not in params:
            raise ValueError(f"missing parameter {k}")
        if params[k] is None and k in BIAS_KEYS:
            continue  # a projection without a bias
        want = (C, C) if k.endswith("_weight") and not k.startswith("norm") else (C,)
        if tuple(np.shape(params[k])) != want:
            raise ValueError(f"{k} must have shape {want}")
    if num_groups < 1 or C % num_groups:
        raise ValueError("num_groups must divide C")
    if num_heads < 1 or C % num_heads:
        raise ValueError("num_heads must divide C")
    return B, C, H, W


def group_norm(x, weight, bias, num_groups: int, eps: float = EPS):
    """GroupNorm with affine (tensortonic problem, prose after the formula).

    Reading (the page is silent on these): group g holds the contiguous
    channels g*C/G .. (g+1)*C/G - 1 over all H*W pixels; the variance is the
    biased one (divide by the element count), computed in two passes; eps is
    added inside the square root; the per-channel affine is applied after
    normalising.

    Returns (GN(x), mean, var) with mean and var of shape (B, G).
    """
    x = _f64(x)
    B, C, H, W = x.shape
    G = num_groups
    xg = x.reshape(B, G, (C // G) * H * W)
    mean = xg.mean(axis=2)
    var = ((xg - mean[:, :, None]) ** 2).mean(axis=2)
    xhat = (xg - mean[:, :, None]) / np.sqrt(var[:, :, None] + eps)
    xhat = xhat.reshape(B, C, H, W)
    y = xhat * _f64(weight)[None, :, None, None] + _f64(bias)[None, :, None, None]
    return y, mean, var


def tokens(img):
    """(B, C, H, W) -> (B, H*W, C) with pixel (i, j) at row i*W + j.

    tensortonic problem, prose ("tokens step") and its first hint
    (flatten the spatial axes, then swap them with channels).
    """
    img = _f64(img)
    B, C, H, W = img.shape
    return img.reshape(B, C, H * W).transpose(0, 2, 1)


def image(tok, H: int, W: int):
    """Inverse of tokens(): (B, H*W, C) -> (B, C, H, W) (tensortonic problem, prose)."""
    tok = _f64(tok)
    B, T, C = tok.shape
    return tok.transpose(0, 2, 1).reshape(B, C, H, W)


def linear(z, weight, bias):
    """z W^T + b, with W stored (out, in) "as in a linear layer" (tensortonic problem, prose).

    bias None: a projection built without a bias (HNDL attention operator,
    "Biases"), i.e. z W^T.
    """
    y = _f64(z) @ _f64(weight).T
    return y if bias is None else y + _f64(bias)


def softmax_keys(S):
    """Softmax along the last (key) axis (tensortonic problem, third hint).

    exp(S - rowmax) / sum exp(S - rowmax): the same value as exp(S)/sum exp(S),
    with the row max taken out so large logits do not overflow.
    """
    S = _f64(S)
    e = np.exp(S - S.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(Q, K, V, num_heads: int):
    """Multi-head attention over tokens, heads concatenated in head order.

    tensortonic problem, formula and prose: head j uses channels j*d ..
    (j+1)*d - 1 of Q, K and V, with d = C/n; its scores are Q_j K_j^T / sqrt(d)
    (the page's formula lost the radical in extraction; its first worked
    example states the scores are divided by sqrt(2) at d = 2); the softmax
    runs over keys; O_j = P_j V_j; heads are concatenated back along channels.

    Q, K, V are (B, T, C); returns (O, P) with O (B, T, C) and P (B, n, T, T).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, T, C = Q.shape
    n = num_heads
    d = C // n
    O = np.empty_like(Q)
    P = np.empty((B, n, T, T))
    for j in range(n):
        sl = slice(j * d, (j + 1) * d)
        S = Q[:, :, sl] @ K[:, :, sl].transpose(0, 2, 1) / np.sqrt(d)
        P[:, j] = softmax_keys(S)
        O[:, :, sl] = P[:, j] @ V[:, :, sl]
    return O, P


def split_heads(M, num_heads: int):
    """(B, T, C) -> (B, n, T, d): head j takes channels j*d .. (j+1)*d - 1."""
    M = _f64(M)
    B, T, C = M.shape
    return M.reshape(B, T, num_heads, C // num_heads).transpose(0, 2, 1, 3)


def merge_heads(Mh):
    """(B, n, T, d) -> (B, T, C), heads concatenated in head order."""
    Mh = _f64(Mh)
    B, n, T, d = Mh.shape
    return Mh.transpose(0, 2, 1, 3).reshape(B, T, n * d)


def qk_norm(Xh, gamma):
    """Per-head query/key normalisation (vit-pytorch simple_vit_with_qk_norm.py,
    class RMSNorm): F.normalize over the head dimension -- x / max(||x||_2, 1e-12)
    -- times sqrt(d) times the learned gamma of the head.  Xh is (B, n, T, d),
    gamma is (n, d)."""
    Xh = _f64(Xh)
    d = Xh.shape[-1]
    nrm = np.sqrt((Xh * Xh).sum(axis=-1, keepdims=True))
    return Xh / np.maximum(nrm, 1e-12) * np.sqrt(d) * _f64(gamma)[None, :, None, :]


def rope_angles(positions, d: int):
    """Rotation angles of the HNDL attention operator ("Rotary embeddings"):
    theta_i = 10000 ** (-2 i / d) for i < d/2 and angle = t * theta_i, built in
    float32 as the page states (theta_i rounded to float32, then one float32
    product).  Returns float64 values of those float32 angles, (len(positions), d/2)."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.float32(10000.0 ** (-2.0 * i / d))
    t = np.asarray(positions, dtype=np.float32)
    return (t[:, None] * theta[None, :]).astype(np.float32).astype(np.float64)


def rope(Xh, positions):
    """Rotary embedding over the full head dimension, rotate-half convention
    (HNDL attention operator, "Rotary embeddings"):
    x * cos(angle) + rotate_half(x) * sin(angle), rotate_half([a, b]) = [-b, a]
    with a, b the two halves of the head; token t of the sequence at position
    t.  Xh is (B, n, T, d) with the tokens listed in ``positions``."""
    Xh = _f64(Xh)
    d = Xh.shape[-1]
    if d % 2:
        raise ValueError("rotary embeddings need an even head size")
    ang = rope_angles(positions, d)                  # (T, d/2)
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=-1)
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=-1)
    a, b = Xh[..., : d // 2], Xh[..., d // 2:]
    rot = np.concatenate([-b, a], axis=-1)
    return Xh * cos + rot * sin


def rel_pos_bias(table, H: int, W: int, rows=None):
    """The [heads, rows, T] additive logit bias of the HNDL attention operator
    ("Relative position bias"): token t sits at row t // W, column t % W; for
    query q and key k, dy = row(q) - row(k) + H - 1, dx = col(q) - col(k) + W - 1,
    and bias[head, q, k] = table[dy * (2W - 1) + dx, head].  table is
    ((2H-1)*(2W-1), heads); rows lists the query tokens (default: all)."""
    table = _f64(table)
    T = H * W
    q = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    k = np.arange(T)
    dy = (q // W)[:, None] - (k // W)[None, :] + (H - 1)
    dx = (q % W)[:, None] - (k % W)[None, :] + (W - 1)
    idx = dy * (2 * W - 1) + dx                      # (R, T)
    return table[idx].transpose(2, 0, 1)             # (heads, R, T)


def check_options(C: int, H: int, W: int, num_heads: int, rel_pos_table, q_norm_gamma,
                  k_norm_gamma, rope_on: bool):
    """Shape rules of the optional steps."""
    d = C // num_heads
    if rel_pos_table is not None and np.shape(rel_pos_table) != ((2 * H - 1) * (2 * W - 1), num_heads):
        raise ValueError("rel_pos_table must be ((2H-1)*(2W-1), num_heads)")
    if (q_norm_gamma is None) != (k_norm_gamma is None):
        raise ValueError("query/key normalisation needs both gammas")
    if q_norm_gamma is not None:
        for g in (q_norm_gamma, k_norm_gamma):
            if np.shape(g) != (num_heads, d):
                raise ValueError("norm gammas must be (num_heads, d)")
    if rope_on and d % 2:
        raise ValueError("rotary embeddings need an even head size")


def attend(Qh, Kh, Vh, scale: float, bias=None):
    """softmax_keys(Qh Kh^T * scale + bias) Vh per head; bias (n, Tq, Tk) or None.
    Returns (O (B, n, Tq, d), P (B, n, Tq, Tk))."""
    S = _f64(Qh) @ _f64(Kh).transpose(0, 1, 3, 2) * scale
    if bias is not None:
        S = S + _f64(bias)[None]
    P = softmax_keys(S)
    return P @ _f64(Vh), P


def forward_stages(x, params, num_groups: int, num_heads: int, rel_pos_table=None,
                   q_norm_gamma=None, k_norm_gamma=None, rope_on: bool = False) -> dict:
    """Every intermediate of the block, in the order of the page's formula.

    Keys: mean, var (B, G); rstd (B, G); Z, Q, K, V, O, Y (B, T, C) -- Q and K
    as they enter the scores, i.e. after the optional normalisation and
    rotation; P (B, n, T, T); out (B, C, H, W).  All float64.
    """
    B, C, H, W = check_args(x, params, num_groups, num_heads)
    check_options(C, H, W, num_heads, rel_pos_table, q_norm_gamma, k_norm_gamma, rope_on)
    p = {k: (None if v is None else _f64(v)) for k, v in params.items()}
    x = _f64(x)
    T, d = H * W, C // num_heads
    gn, mean, var = group_norm(x, p["norm_weight"], p["norm_bias"], num_groups)
    Z = tokens(gn)
    Q = linear(Z, p["q_weight"], p["q_bias"])
    K = linear(Z, p["k_weight"], p["k_bias"])
    V = linear(Z, p["v_weight"], p["v_bias"])
    plain = rel_pos_table is None and q_norm_gamma is None and not rope_on
    if plain:
        O, P = attention(Q, K, V, num_heads)
    else:
        Qh, Kh, Vh = (split_heads(M, num_heads) for M in (Q, K, V))
        if q_norm_gamma is not None:
            Qh, Kh = qk_norm(Qh, q_norm_gamma), qk_norm(Kh, k_norm_gamma)
        if rope_on:
            Qh, Kh = rope(Qh, np.arange(T)), rope(Kh, np.arange(T))
        scale = 1.0 if q_norm_gamma is not None else 1.0 / np.sqrt(d)
        bias = None if rel_pos_table is None else rel_pos_bias(rel_pos_table, H, W)
        Oh, P = attend(Qh, Kh, Vh, scale, bias)
        Q, K, O = merge_heads(Qh), merge_heads(Kh), merge_heads(Oh)
    Y = linear(O, p["out_weight"], p["out_bias"])
    out = x + image(Y, H, W)
    return dict(mean=mean, var=var, rstd=1.0 / np.sqrt(var + EPS),
                Z=Z, Q=Q, K=K, V=V, P=P, O=O, Y=Y, out=out)


def forward(x, params, num_groups: int, num_heads: int, **options) -> np.ndarray:
    """out = x + image([O_1..O_n] Wo^T + bo), float64, shape (B, C, H, W).

    options: rel_pos_table, q_norm_gamma, k_norm_gamma, rope_on (see
    forward_stages)."""
    return forward_stages(x, params, num_groups, num_heads, **options)["out"]


def forward_pixels(x, params, num_groups: int, num_heads: int, b: int, rows, rel_pos_table=None,
                   q_norm_gamma=None, k_norm_gamma=None, rope_on: bool = False):
    """out[b, :, i, j] for the token rows t = i*W + j listed in ``rows``.

    The same definition as forward(), evaluated for a few query rows of one
    sample: GroupNorm statistics and K, V need every pixel of sample b, but Q,
    the score rows, the softmax and the output projection are only formed for
    the requested rows (each output pixel depends on its own query row only).
    Returns an array of shape (C, len(rows)).
    """
    B, C, H, W = check_args(x, params, num_groups, num_heads)
    check_options(C, H, W, num_heads, rel_pos_table, q_norm_gamma, k_norm_gamma, rope_on)
    p = {k: (None if v is None else _f64(v)) for k, v in params.items()}
    rows = np.asarray(rows, dtype=np.int64)
    T = H * W
    xb = _f64(x)[b:b + 1]
    gn, _, _ = group_norm(xb, p["norm_weight"], p["norm_bias"], num_groups)
    Z = tokens(gn)                                   # (1, T, C)
    K = linear(Z, p["k_weight"], p["k_bias"])
    V = linear(Z, p["v_weight"], p["v_bias"])
    Qr = linear(Z[:, rows], p["q_weight"], p["q_bias"])
    n = num_heads
    d = C // n
    Qh, Kh, Vh = split_heads(Qr, n), split_heads(K, n), split_heads(V, n)
    if q_norm_gamma is not None:
        Qh, Kh = qk_norm(Qh, q_norm_gamma), qk_norm(Kh, k_norm_gamma)
    if rope_on:
        Qh, Kh = rope(Qh, rows), rope(Kh, np.arange(T))
    scale = 1.0 if q_norm_gamma is not None else 1.0 / np.sqrt(d)
    bias = None if rel_pos_table is None else rel_pos_bias(rel_pos_table, H, W, rows)
    Oh, _ = attend(Qh, Kh, Vh, scale, bias)
    Yr = linear(merge_heads(Oh)[0], p["out_weight"], p["out_bias"])   # (R, C)
    xr = xb[0].reshape(C, T)[:, rows]
    return xr + Yr.T
