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
    """z W^T + b, with W stored (out, in) "as in a linear layer" (tensortonic problem, prose)."""
    return _f64(z) @ _f64(weight).T + _f64(bias)


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


def forward_stages(x, params, num_groups: int, num_heads: int) -> dict:
    """Every intermediate of the block, in the order of the page's formula.

    Keys: mean, var (B, G); rstd (B, G); Z, Q, K, V, O, Y (B, T, C);
    P (B, n, T, T); out (B, C, H, W).  All float64.
    """
    B, C, H, W = check_args(x, params, num_groups, num_heads)
    p = {k: _f64(v) for k, v in params.items()}
    x = _f64(x)
    gn, mean, var = group_norm(x, p["norm_weight"], p["norm_bias"], num_groups)
    Z = tokens(gn)
    Q = linear(Z, p["q_weight"], p["q_bias"])
    K = linear(Z, p["k_weight"], p["k_bias"])
    V = linear(Z, p["v_weight"], p["v_bias"])
    O, P = attention(Q, K, V, num_heads)
    Y = linear(O, p["out_weight"], p["out_bias"])
    out = x + image(Y, H, W)
    return dict(mean=mean, var=var, rstd=1.0 / np.sqrt(var + EPS),
                Z=Z, Q=Q, K=K, V=V, P=P, O=O, Y=Y, out=out)


def forward(x, params, num_groups: int, num_heads: int) -> np.ndarray:
    """out = x + image([O_1..O_n] Wo^T + bo), float64, shape (B, C, H, W)."""
    return forward_stages(x, params, num_groups, num_heads)["out"]


def forward_pixels(x, params, num_groups: int, num_heads: int, b: int, rows):
    """out[b, :, i, j] for the token rows t = i*W + j listed in ``rows``.

    The same definition as forward(), evaluated for a few query rows of one
    sample: GroupNorm statistics and K, V need every pixel of sample b, but Q,
    the score rows, the softmax and the output projection are only formed for
    the requested rows (each output pixel depends on its own query row only).
    Returns an array of shape (C, len(rows)).
    """
    B, C, H, W = check_args(x, params, num_groups, num_heads)
    p = {k: _f64(v) for k, v in params.items()}
    rows = np.asarray(rows, dtype=np.int64)
    xb = _f64(x)[b:b + 1]
    gn, _, _ = group_norm(xb, p["norm_weight"], p["norm_bias"], num_groups)
    Z = tokens(gn)[0]                         # (T, C)
    K = linear(Z, p["k_weight"], p["k_bias"])
    V = linear(Z, p["v_weight"], p["v_bias"])
    Qr = linear(Z[rows], p["q_weight"], p["q_bias"])
    n = num_heads
    d = C // n
    Or = np.empty_like(Qr)
    for j in range(n):
        sl = slice(j * d, (j + 1) * d)
        S = Qr[:, sl] @ K[:, sl].T / np.sqrt(d)
        Or[:, sl] = softmax_keys(S) @ V[:, sl]
    Yr = linear(Or, p["out_weight"], p["out_bias"])      # (R, C)
    xr = xb[0].reshape(C, H * W)[:, rows]
    return xr + Yr.T
