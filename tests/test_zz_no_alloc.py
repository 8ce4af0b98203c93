"""ssa_forward_noalloc, the entry point that allocates nothing (its workspace
is the library's static scratch), against ssa_forward with a caller
workspace, through the C ABI: two calls in a row on one GPU, the second with
a smaller problem (the scratch keeps the first call's contents), each output
equal to ssa_forward's bit for bit and within the bf16 bar of the oracle on
sampled pixels."""
import numpy as np
import pytest
import torch

import oracle as ORA
import spatial_self_attention_amd as ssa
from spatial_self_attention_amd.inputs import WORKLOADS, draw, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def noalloc(xg, pg, wl, out):
    B, C, H, W = xg.shape
    ptrs = [0 if pg[k] is None else pg[k].data_ptr() for k in ssa.PARAM_ORDER]
    stream = torch.cuda.current_stream(xg.device).cuda_stream
    return ssa.ssa_forward_noalloc(xg.data_ptr(), out.data_ptr(), ptrs, B, C, H, W,
                                   wl.num_groups, wl.num_heads, ssa.dtype_code(xg.dtype), stream)


def test_noalloc_matches_forward_twice():
    # the largest workload first (97 MB of scratch), then a smaller problem of
    # another shape, dtype path and head size
    cases = ((WORKLOADS[4], 1004, 2), (WORKLOADS[3].replace(B=1, H=20, W=26), 7, 1))
    for wl, seed, nb in cases:
        x, p = draw(wl, seed)
        xg = x.to(DEV)
        pg = {k: v.to(DEV) for k, v in p.items()}
        print(f"[gpu] noalloc {wl.name} B={wl.B} {wl.H}x{wl.W}", flush=True)
        ref = ssa.spatial_self_attention(xg, pg, wl.num_groups, wl.num_heads)
        out = torch.full_like(xg, float("nan"))
        st = noalloc(xg, pg, wl, out)
        assert st == 0, ssa.ssa_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        # and the oracle's bar on sampled pixels of the first and last sample
        x64, p64 = to_f64(x, p)
        og = out.double().cpu().numpy().reshape(wl.B, wl.C, wl.T)
        rng = np.random.default_rng(seed)
        for b in sorted({0, wl.B - 1})[:nb]:
            rows = np.unique(np.concatenate([[0, wl.T - 1], rng.integers(0, wl.T, 4)]))
            want = ORA.forward_pixels(x64, p64, wl.num_groups, wl.num_heads, b, rows)
            e = float(np.max(np.abs(og[b][:, rows] - want))) / float(np.max(np.abs(want)))
            print(f"  sampled err {e:.3e}", flush=True)
            assert e <= 2e-2


def test_noalloc_fp32_after_bf16():
    wl = WORKLOADS[0]
    x, p = draw(wl, 17)
    xg = x.to(DEV)
    pg = {k: v.to(DEV) for k, v in p.items()}
    ref = ssa.spatial_self_attention(xg, pg, wl.num_groups, wl.num_heads)
    out = torch.full_like(xg, float("nan"))
    assert noalloc(xg, pg, wl, out) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    want = ORA.forward(*to_f64(x, p), wl.num_groups, wl.num_heads)
    assert float(np.max(np.abs(out.double().cpu().numpy() - want))) <= 1e-4
