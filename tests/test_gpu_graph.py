"""The block replayed from a captured HIP graph.

Callers capture ssa_forward / ssa_forward_ex into graphs (bench.py times the
step and its stages that way).  A graph is captured once, then replayed several times with
the inputs changed in place between replays and an eager call (own output and
workspace) and a synchronisation in between; every replay must equal the eager
result bit for bit (the same kernels on the same inputs).
"""
import pytest
import torch

import spatial_self_attention_amd as ssa
from spatial_self_attention_amd.inputs import WORKLOADS, Workload, draw, draw_options

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    (WORKLOADS[2].replace(B=2), {}),                                  # bf16 d64, plain
    (WORKLOADS[1], {}),                     # bf16 d128, B n >= CUs: the 8-wave attention path
    (Workload("bf16 d64 12x13", "bf16", 2, 128, 12, 13, 8, 2),
     dict(rel_pos=True, qk_norm=True, rope=True)),                    # every optional step
    (WORKLOADS[0], {}),                                               # fp32
    (WORKLOADS[3], {}),                     # LDM level-1: d64, long sequences, one-block kernel
    (WORKLOADS[4], {}),                     # high-res: the two-block attention kernel
]


@pytest.mark.parametrize("wl,flags", CASES, ids=["bf16-d64", "bf16-d128-8wave", "bf16-options", "fp32",
                                                 "bf16-ldm-level1", "bf16-high-res"])
def test_graph_replays_equal_eager(wl, flags):
    x, p = draw(wl, 61)
    xg = x.to(DEV)
    pg = {k: v.to(DEV) for k, v in p.items()}
    opts = None
    if flags:
        od = draw_options(wl, 61, **flags)
        odg = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in od.items()}
        opts = ssa.make_options(xg, wl.num_heads, odg["rel_pos_table"], odg["q_norm_gamma"],
                                odg["k_norm_gamma"], odg["rope"])
    print(f"[gpu] graph {wl.name} dtype={wl.dtype} B={wl.B} opts={flags}", flush=True)
    out_g = torch.empty_like(xg)
    ws_g = ssa.workspace_for(xg, wl.num_groups, wl.num_heads)
    out_e = torch.empty_like(xg)
    ws_e = ssa.workspace_for(xg, wl.num_groups, wl.num_heads)
    # warm the library up on the capture's buffers, then capture
    ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out_g, ws_g, options=opts)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out_g, ws_g, options=opts)
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV).manual_seed(7)
    for r in range(3):
        # new inputs in place (the graph reads xg), an eager call, then the replay
        xg.copy_((torch.randn(xg.shape, generator=gen, device=DEV) * (1.0 + r)).to(xg.dtype))
        out_g.fill_(float("nan"))
        ssa.forward_into(xg, pg, wl.num_groups, wl.num_heads, out_e, ws_e, options=opts)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(out_g).all(), f"replay {r}"
        assert torch.equal(out_g, out_e), f"replay {r} differs from the eager call"
