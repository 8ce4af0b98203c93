"""A seeded sweep of small random shapes against the fp64 oracle.

The other parity tests pick their shapes by hand; this one draws 40 from a
fixed seed so that sizes nobody chose get checked too: both dtypes, every
supported bf16 head size, odd image sizes (ragged token tiles, grid rows not a
multiple of any tile), group counts that do not divide the heads, the optional
steps in random combinations and absent biases.  The list is fixed (seeded),
so a failure names a reproducible case.  Tolerances as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle as ORA
import spatial_self_attention_amd as ssa
from spatial_self_attention_amd.inputs import Workload, draw, draw_options, options_f64, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _cases(n_cases=40, seed=20241202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        if dtype == "bf16":
            d = int(rng.choice([32, 64, 96, 128]))
        else:
            d = int(rng.choice([4, 8, 12, 16, 32, 48, 64, 100, 128]))
        n = int(rng.integers(1, 4))
        C = n * d
        divisors = [g for g in range(1, min(C, 32) + 1) if C % g == 0]
        G = int(rng.choice(divisors))
        H, W = int(rng.integers(1, 21)), int(rng.integers(1, 21))
        B = int(rng.integers(1, 4))
        flags = dict(rel_pos=bool(rng.random() < 0.3), qk_norm=bool(rng.random() < 0.3),
                     rope=bool(rng.random() < 0.3) and d % 2 == 0)
        drop = tuple(k for k in ("q_bias", "k_bias", "v_bias", "out_bias") if rng.random() < 0.15)
        out.append((Workload(f"sweep{i}", dtype, B, C, H, W, G, n), flags, drop))
    return out


CASES = _cases()


@pytest.mark.parametrize("wl,flags,drop", CASES, ids=[c[0].name for c in CASES])
def test_random_shape(wl, flags, drop):
    x, p = draw(wl, 300)
    for k in drop:
        p[k] = None
    opts = draw_options(wl, 300, **flags)
    print(f"[gpu] {wl.name} dtype={wl.dtype} B={wl.B} C={wl.C} H={wl.H} W={wl.W} "
          f"G={wl.num_groups} n={wl.num_heads} opts={flags} drop={drop}", flush=True)
    dev = lambda t: None if t is None else t.to(DEV)
    out = ssa.spatial_self_attention(
        x.to(DEV), {k: dev(v) for k, v in p.items()}, wl.num_groups, wl.num_heads,
        rel_pos_table=dev(opts["rel_pos_table"]), q_norm_gamma=dev(opts["q_norm_gamma"]),
        k_norm_gamma=dev(opts["k_norm_gamma"]), rope=opts["rope"])
    torch.cuda.synchronize()
    want = ORA.forward(*to_f64(x, p), wl.num_groups, wl.num_heads, **options_f64(opts))
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    e = float(np.max(np.abs(got - want)))
    if wl.dtype == "bf16":
        e /= max(float(np.max(np.abs(want))), 1e-30)
    print(f"  err {e:.3e}", flush=True)
    assert e <= TOL[wl.dtype]
