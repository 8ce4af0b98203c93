"""The fused projection + attention stage (SSA_STAGE_QKV_ATTENTION) on the GPU.

Where ssa_uses_fused_stage() holds, ssa_forward runs stages 0, 4, 3 instead of
0, 1, 2, 3.  Stage 4 forms the same bf16 Q, K and V as stage 1 (same products
in the same order, same bias, scale and rounding) and runs the attention
kernel's operations on them in the same order, so its O must equal the O of
stages 1 + 2 bit for bit, and the block's output must be the same either way.
Full-size cases are also checked against the fp64 oracle on sampled pixels
(every head of the sampled tokens), plain and on stressed inputs.
"""
import numpy as np
import pytest
import torch

import oracle as ORA
import spatial_self_attention_amd as ssa
from spatial_self_attention_amd.inputs import WORKLOADS, Workload, draw, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2  # bf16 normwise max-relative, as in test_gpu_parity


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _fill(wl):
    """wl with enough samples that every compute unit gets a (sample, head)."""
    need = -(-_cus() // wl.num_heads)
    return wl if wl.B >= need else wl.replace(B=need)


CASES = [
    WORKLOADS[1],                                          # T = 196: 7 key blocks, partial tail
    WORKLOADS[1].replace(H=16, W=16),                      # T = 256: 8 blocks
    WORKLOADS[1].replace(H=14, W=16),                      # T = 224: 7 blocks, no partial block
    WORKLOADS[1].replace(H=10, W=20),                      # T = 200
    Workload("C256 n2 14x14", "bf16", 128, 256, 14, 14, 32, 2),
    Workload("C1536 n12 14x14", "bf16", 22, 1536, 14, 14, 32, 12),  # largest C
]
IDS = ["c196", "t256", "t224", "t200", "c256", "c1536"]


def _setup(wl, seed, stress=False, drop=()):
    x, p = draw(wl, seed, stress=stress)
    for k in drop:
        p[k] = None
    xg = x.to(DEV)
    pg = {k: (None if v is None else v.to(DEV)) for k, v in p.items()}
    return x, p, xg, pg


def _o_region(ws, wl):
    lay = ssa.ssa_get_workspace_layout(wl.B, wl.C, wl.H, wl.W, wl.num_groups, wl.num_heads,
                                       ssa.SSA_BF16)
    n = wl.B * wl.T * wl.C * 2
    return ws[lay["o"]: lay["o"] + n].clone()


def _run_stages(xg, pg, wl, stages):
    out = torch.full_like(xg, float("nan"))
    ws = ssa.workspace_for(xg, wl.num_groups, wl.num_heads)
    ws.fill_(0xFF)
    for stage in stages:
        ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out, ws, stage=stage)
    torch.cuda.synchronize()
    return out, ws


@pytest.mark.parametrize("drop", [(), ("q_bias", "k_bias", "v_bias")], ids=["bias", "nobias"])
@pytest.mark.parametrize("wl", CASES, ids=IDS)
def test_fused_equals_separate_stages(wl, drop):
    wl = _fill(wl)
    assert ssa.ssa_uses_fused_stage(wl.B, wl.C, wl.H, wl.W, wl.num_groups, wl.num_heads,
                                    ssa.SSA_BF16)
    x, p, xg, pg = _setup(wl, 71, drop=drop)
    print(f"[gpu] fused {wl.name} B={wl.B} C={wl.C} {wl.H}x{wl.W} n={wl.num_heads} drop={drop}",
          flush=True)
    out_sep, ws_sep = _run_stages(xg, pg, wl, ("gn_stats", "qkv", "attention", "out_proj"))
    out_fus, ws_fus = _run_stages(xg, pg, wl, ("gn_stats", "qkv_attention", "out_proj"))
    assert torch.isfinite(out_fus).all()
    assert torch.equal(_o_region(ws_fus, wl), _o_region(ws_sep, wl)), "O differs"
    assert torch.equal(out_fus, out_sep)
    ref = ssa.spatial_self_attention(xg, pg, wl.num_groups, wl.num_heads)
    torch.cuda.synchronize()
    assert torch.equal(ref, out_fus)
    assert ssa.forward_stages(xg, wl.num_groups, wl.num_heads) == (
        "gn_stats", "qkv_attention", "out_proj")


@pytest.mark.parametrize("stress", [False, True], ids=["plain", "stressed"])
@pytest.mark.parametrize("wl", CASES[:2] + CASES[4:], ids=IDS[:2] + IDS[4:])
def test_fused_full_size_sampled_oracle(wl, stress):
    wl = _fill(wl)
    x, p, xg, pg = _setup(wl, 81, stress=stress)
    print(f"[gpu] fused oracle {wl.name} B={wl.B} C={wl.C} {wl.H}x{wl.W} stress={stress}",
          flush=True)
    out = ssa.spatial_self_attention(xg, pg, wl.num_groups, wl.num_heads)
    torch.cuda.synchronize()
    og = out.double().cpu().numpy().reshape(wl.B, wl.C, wl.T)
    assert np.isfinite(og).all()
    x64, p64 = to_f64(x, p)
    rng = np.random.default_rng(wl.T + wl.C)
    worst = 0.0
    for b in sorted({0, wl.B // 2, wl.B - 1}):
        rows = np.unique(np.concatenate([[0, wl.T - 1], rng.integers(0, wl.T, 5)]))
        want = ORA.forward_pixels(x64, p64, wl.num_groups, wl.num_heads, b, rows)
        e = float(np.max(np.abs(og[b][:, rows] - want))) / float(np.max(np.abs(want)))
        worst = max(worst, e)
    print(f"  sampled err {worst:.3e}", flush=True)
    assert worst <= TOL


def test_fused_stage_rejected_where_unavailable():
    wl = WORKLOADS[2].replace(B=2)  # d = 64
    assert not ssa.ssa_uses_fused_stage(wl.B, wl.C, wl.H, wl.W, wl.num_groups, wl.num_heads,
                                        ssa.SSA_BF16)
    _, _, xg, pg = _setup(wl, 5)
    out = torch.empty_like(xg)
    ws = ssa.workspace_for(xg, wl.num_groups, wl.num_heads)
    with pytest.raises(ssa.SSAValueError):
        ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out, ws, stage="qkv_attention")
    assert ssa.forward_stages(xg, wl.num_groups, wl.num_heads) == (
        "gn_stats", "qkv", "attention", "out_proj")
