"""The attention stage alone on long sequences (bf16, d = 64, T >= 1024),
covering each kernel shape the stage picks there: the two-query-block kernel
with 512-query work-groups (key tiles of 128) or 256-query work-groups (key
tiles of 64: 8-wave work-groups that split the keys in halves and merge in
LDS when the sequence is a multiple of 128 (T = 9216, 8320), two 4-wave
work-groups per CU otherwise (T = 9215, 9280)), the same 8-wave kernel with
the tiles of a partial last round cut into 4, 7 or 8 key ranges whose
partial results a second kernel merges (one round of tiles and a last round
filling at most half the CUs), and the one-block kernel when the query
tiles are too few to fill whole rounds of the CUs (the choice assumes
MI355X's 256 CUs); and six seeded random shapes for the key-splitting kernel.

Seeded Q, K, V (spatial_self_attention_amd.inputs.draw_qkv) are written into
the workspace in the layouts the stage reads, the stage runs alone, and O is
compared with the oracle's per-head softmax(Q K^T) V in fp64 on the same
values (scores 2^(q.k) = e^(q.k ln 2): the stored q carries the score scale),
over every row for the smaller shapes and sampled rows (each query tile's
first and last, and random ones) for the larger ones.  Ragged key tiles
(T % 128 = 1, T % 64 = 63) and ragged last query tiles are included; scores
both peaked and rising along the keys (the running max raised in every key
block, early keys' weights underflowing).
Tolerance: max |gpu - oracle| / max |oracle| <= 1e-2 (bf16 probabilities and
output).
"""
import numpy as np
import pytest
import torch

import oracle as ORA
import spatial_self_attention_amd as ssa
from spatial_self_attention_amd.inputs import draw_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-2


def vt_cols(Tp):
    """Column of token t in a bf16 V^T row: bits 2 and 3 of t swapped."""
    t = np.arange(Tp)
    return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1)


def run_attention(B, n, H, W, seed, kind):
    d = 64
    C, T = n * d, H * W
    q, k, v = draw_qkv(B, n, T, d, seed, kind)
    x = torch.zeros((B, C, H, W), dtype=torch.bfloat16, device=DEV)
    params = {key: torch.zeros((C, C) if key.endswith("_weight") and key != "norm_weight" else (C,),
                               dtype=torch.bfloat16, device=DEV) for key in ssa.PARAM_ORDER}
    ws = ssa.workspace_for(x, 1, n)
    ws.fill_(0xFF)  # NaN patterns everywhere, including V^T's padding columns
    lay = ssa.ssa_get_workspace_layout(B, C, H, W, 1, n, ssa.SSA_BF16)
    Tp = lay["t_pad"]

    def put(name, t):
        raw = t.contiguous().view(torch.uint8).reshape(-1)
        ws[lay[name]: lay[name] + raw.numel()] = raw.to(DEV)

    put("q", q)
    put("k", k)
    vt = torch.full((B, n, d, Tp), float("nan"), dtype=torch.bfloat16)
    vt[..., torch.from_numpy(vt_cols(Tp)[:T])] = v.transpose(2, 3)
    put("vt", vt)
    out = torch.empty_like(x)
    print(f"[gpu] attention B={B} n={n} H={H} W={W} T={T} kind={kind} seed={seed}", flush=True)
    ssa.forward_into(x, params, 1, n, out, ws, stage="attention")
    torch.cuda.synchronize()
    raw = ws[lay["o"]: lay["o"] + B * T * C * 2].cpu()
    o = raw.view(torch.bfloat16).reshape(B, T, n, d).permute(0, 2, 1, 3).double().numpy()
    return q, k, v, o


CASES = [
    # (B, n, H, W, rows sampled per head or None for all)
    (1, 5, 33, 40, None),     # one-block kernel; T % 128 = 40
    (4, 5, 64, 64, 64),       # the LDM level-1 workload's shape: 320 tiles of 256, the last
                              # 64 each cut into 4 key ranges
    (2, 9, 64, 64, 40),       # 288 tiles: the last 32 in 8 key ranges of 2 tile pairs
    (1, 17, 66, 64, 40),      # 289 tiles, T % 256 = 128: the last 33 in 7 uneven key ranges
    (1, 89, 32, 32, 24),      # 356 tiles: the last 100 in 2 key ranges
    (1, 81, 32, 32, 24),      # 324 tiles: the last 68 in 3
    (1, 75, 32, 32, 24),      # 300 tiles: the last 44 in 5
    (1, 74, 32, 32, 24),      # 296 tiles: the last 40 in 6
    (1, 5, 32, 32, None),     # 20 tiles: one-block kernel
    (1, 32, 63, 63, 40),      # 256 query tiles of 512: T % 128 = 1, last tile 385 rows
    (2, 16, 64, 64, 48),      # 256 query tiles of 512, even sizes
    (2, 10, 95, 97, 40),      # 720 query tiles of 256: T % 64 = 63
    (2, 10, 96, 96, 40),      # the high-resolution workload's shape: 720 tiles of 256, each
                              # split over the keys by the halves of one work-group
    (2, 10, 80, 104, 40),     # 660 such tiles, the last one of each head 128 rows
    (2, 10, 80, 116, 40),     # T % 128 = 64: two 4-wave work-groups per CU, full key tiles
]


def _random_cases(n_cases=6, seed=20261202):
    """Seeded shapes nobody chose for the key-splitting kernel: T = 128 m in
    [1024, 8192] as an H x W grid, at least one round of 256-query tiles on
    256 CUs (some with the last round cut into key ranges)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n_cases:
        T = 128 * int(rng.integers(8, 65))
        widths = [w for w in range(8, 257) if T % w == 0 and T // w >= 4]
        W = int(rng.choice(widths))
        B, n = int(rng.integers(1, 4)), int(rng.integers(1, 31))
        if B * n * ((T + 255) // 256) >= 256:
            out.append((B, n, T // W, W, 16))
    return out


RANDOM_CASES = _random_cases()


def check_long(case, kind):
    B, n, H, W, per_head = case
    T = H * W
    q, k, v, o = run_attention(B, n, H, W, 40 + n + H, kind)
    assert np.isfinite(o).all()
    rng = np.random.default_rng(T)
    worst = 0.0
    for b in range(B):
        if per_head is None:
            rows = np.arange(T)
        else:  # the first and last rows of every 512-query tile, and random ones
            ends = np.concatenate([np.arange(0, T, 256), np.minimum(np.arange(255, T + 255, 256), T - 1)])
            rows = np.unique(np.concatenate([ends, rng.integers(0, T, per_head)]))
        qh = q[b:b + 1, :, rows].double().numpy()
        want, _ = ORA.attend(qh, k[b:b + 1].double().numpy(), v[b:b + 1].double().numpy(), np.log(2.0))
        got = o[b:b + 1, :, rows]
        e = float(np.max(np.abs(got - want)) / np.max(np.abs(want)))
        worst = max(worst, e)
    print(f"  err {worst:.3e}", flush=True)
    assert worst <= TOL


@pytest.mark.parametrize("kind", ["peaked", "ramp"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}-n{c[1]}-{c[2]}x{c[3]}")
def test_attention_stage_long(case, kind):
    check_long(case, kind)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: f"B{c[0]}-n{c[1]}-{c[2]}x{c[3]}")
def test_attention_stage_long_random(case):
    check_long(case, "ramp" if case[1] % 2 else "peaked")
