"""The C ABI without a GPU: the library loads, exports every entry point
include/ssa.h declares, sizes its workspace, and rejects bad arguments on the
host before anything is launched.

Pointers passed here are fake (never dereferenced): every case returns an
error status from host-side validation, or is an empty input that launches
nothing.
"""
import ctypes
import os
import re

import pytest

import spatial_self_attention_amd as ssa
from spatial_self_attention_amd import _binding as bnd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")

S = {name: code for code, name in bnd.STATUS_NAMES.items()}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = ssa.lib()
    names = declared_functions()
    assert set(names) == set(bnd.EXPORTS), names
    for name in names:
        assert hasattr(L, name), f"libssa.so does not export {name}"


def test_status_strings():
    for code in list(bnd.STATUS_NAMES) + [99, -1]:
        s = ssa.ssa_status_string(code)
        assert isinstance(s, str) and s
    assert ssa.ssa_status_string(0) == "ok"


def _layout_expect(B, C, H, W, G, n, esize):
    T = H * W
    d = C // n
    dp = d if esize == 4 else -(-d // 32) * 32      # bf16 heads padded to a multiple of 32
    Tp = (T + 63) // 64 * 64
    fuse = esize == 2 and C % 64 == 0 and T % 4 == 0 and d in (16, 32, 64, 128)
    # partial (O, m, l) of the key ranges of a partial last round of 256-query
    # tiles (bf16 heads padded to 64, T >= 1024, T % 128 == 0; sized for 256
    # compute units, the count assumed where no device is visible): r tiles
    # filling at most half the units, each cut into min(256 // r, 8, T // 128)
    # ranges of 4 waves x 64 lanes x 68 floats
    part = 0
    t256 = B * n * -(-T // 256)
    r = t256 % 256
    if esize == 2 and dp == 64 and T >= 1024 and T % 128 == 0 and t256 >= 256 and 0 < 2 * r <= 256:
        part = r * min(256 // r, 8, T // 128) * 4 * 64 * 68 * 4
    return {
        "gn_stats": B * G * 8, "gn_coef": B * C * 8,
        "q": B * n * T * dp * esize, "k": B * n * T * dp * esize,
        "vt": B * n * dp * Tp * esize, "o": B * T * C * esize,
        # rotary (cos, sin) table where the projection epilogue runs the
        # optional steps, else fp32 Q and K for the separate pass (bf16 only)
        "rope": T * (d // 2) * 8 if fuse else 0,
        "qk32": 2 * B * T * C * 4 if (esize == 2 and not fuse) else 0,
        "attn_part": part,
        "d_pad": dp,
    }


@pytest.mark.parametrize("shape", [
    (1, 64, 8, 8, 8, 2, ssa.SSA_F32),
    (64, 512, 14, 14, 32, 4, ssa.SSA_BF16),
    (16, 512, 16, 16, 32, 8, ssa.SSA_BF16),
    (4, 320, 64, 64, 32, 5, ssa.SSA_BF16),
    (2, 640, 96, 96, 32, 10, ssa.SSA_BF16),
    (2, 4, 1, 1, 4, 2, ssa.SSA_F32),
    (1, 2, 2, 3, 1, 1, ssa.SSA_F32),
    (2, 4, 1, 1, 4, 2, ssa.SSA_BF16),      # d = 2, padded to 32
    (2, 192, 8, 8, 8, 4, ssa.SSA_BF16),    # d = 48, padded to 64
    (2, 128, 8, 8, 8, 8, ssa.SSA_BF16),    # d = 16, padded to 32
    (2, 576, 64, 64, 32, 9, ssa.SSA_BF16),   # 288 tiles: the last 32 in 8 key ranges
    (1, 1088, 66, 64, 32, 17, ssa.SSA_BF16), # 289 tiles: the last 33 in 7 key ranges
    (3, 640, 64, 64, 32, 10, ssa.SSA_BF16),  # 480 tiles: a last round above half the CUs
])
def test_workspace_layout(shape):
    B, C, H, W, G, n, dt = shape
    lay = ssa.ssa_get_workspace_layout(B, C, H, W, G, n, dt)
    assert lay["total"] == ssa.ssa_workspace_size(B, C, H, W, G, n, dt)
    esize = 4 if dt == ssa.SSA_F32 else 2
    want = _layout_expect(B, C, H, W, G, n, esize)
    assert lay["d_pad"] == want.pop("d_pad")
    want["gn_partial"] = B * G * lay["gn_splits"] * 16
    order = ["gn_partial", "gn_stats", "gn_coef", "q", "k", "vt", "o", "rope", "qk32", "attn_part"]
    for a, b in zip(order, order[1:]):
        assert lay[a] % 256 == 0
        assert lay[a] + want[a] <= lay[b], (a, b)
    assert lay["attn_part"] + want["attn_part"] <= lay["total"]
    # regions of zero bytes take no space: the total is the end of the last non-empty one
    assert lay["total"] - (lay["attn_part"] + want["attn_part"]) < 256
    assert lay["t_pad"] % 64 == 0 and lay["t_pad"] >= H * W
    assert lay["gn_splits"] >= 1
    # every chunk of a segment is non-empty
    L = (C // G) * H * W
    assert (lay["gn_splits"] - 1) * -(-L // lay["gn_splits"]) < L


def test_workspace_size_zero_when_rejected_or_empty():
    assert ssa.ssa_workspace_size(1, 6, 2, 2, 4, 2, ssa.SSA_F32) == 0     # 4 does not divide 6
    assert ssa.ssa_workspace_size(1, 256, 2, 2, 8, 1, ssa.SSA_BF16) == 0  # d = 256
    assert ssa.ssa_workspace_size(0, 64, 8, 8, 8, 2, ssa.SSA_F32) == 0    # empty
    assert ssa.ssa_workspace_size(1, 64, 8, 8, 8, 2, 5) == 0              # dtype


class Fake:
    """Distinct, 256-byte aligned fake device addresses, far apart."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes=1 << 30):
        p = self.next
        self.next += (nbytes + (1 << 20)) // 256 * 256 + 256
        return p


def call(status_fn="ssa_forward", stage=None, **kw):
    B, C, H, W, G, n, dt = kw["shape"]
    fake = Fake()
    ptr = {k: fake() for k in ["x", "out", "ws"] + list(bnd.PARAM_ORDER)}
    ptr.update(kw.get("ptr", {}))
    ws_bytes = kw.get("ws_bytes", ssa.ssa_workspace_size(B, C, H, W, G, n, dt) or 1 << 20)
    params = [ptr[k] for k in bnd.PARAM_ORDER]
    if status_fn == "ssa_forward":
        return ssa.ssa_forward(ptr["x"], ptr["out"], params, B, C, H, W, G, n, dt,
                               ptr["ws"], ws_bytes, 0)
    return ssa.ssa_forward_stage(stage, ptr["x"], ptr["out"], params, B, C, H, W, G, n, dt,
                                 ptr["ws"], ws_bytes, 0)


OK_SHAPE = (2, 64, 4, 4, 8, 2, ssa.SSA_BF16)


@pytest.mark.parametrize("case,kw,want", [
    ("bad dtype", dict(shape=(2, 64, 4, 4, 8, 2, 3)), "SSA_E_DTYPE"),
    ("C = 0", dict(shape=(2, 0, 4, 4, 1, 1, ssa.SSA_F32)), "SSA_E_SHAPE"),
    ("negative B", dict(shape=(-1, 64, 4, 4, 8, 2, ssa.SSA_F32)), "SSA_E_SHAPE"),
    ("negative H", dict(shape=(1, 64, -4, 4, 8, 2, ssa.SSA_F32)), "SSA_E_SHAPE"),
    ("G does not divide C", dict(shape=(2, 64, 4, 4, 7, 2, ssa.SSA_F32)), "SSA_E_CONSTRAINT"),
    ("n does not divide C", dict(shape=(2, 64, 4, 4, 8, 3, ssa.SSA_F32)), "SSA_E_CONSTRAINT"),
    ("G = 0", dict(shape=(2, 64, 4, 4, 0, 2, ssa.SSA_F32)), "SSA_E_CONSTRAINT"),
    ("n = 0", dict(shape=(2, 64, 4, 4, 8, 0, ssa.SSA_F32)), "SSA_E_CONSTRAINT"),
    ("bf16 d = 136", dict(shape=(2, 272, 4, 4, 8, 2, ssa.SSA_BF16)), "SSA_E_UNSUPPORTED"),
    ("fp32 d = 256", dict(shape=(2, 256, 4, 4, 8, 1, ssa.SSA_F32)), "SSA_E_UNSUPPORTED"),
    ("too many elements", dict(shape=(1 << 20, 512, 64, 64, 32, 4, ssa.SSA_BF16)),
     "SSA_E_UNSUPPORTED"),
    # the size limit is exact: 3*B*T*C = 2,147,352,576 passes (and stops at the
    # workspace check: nothing launches), one more sample does not
    ("largest accepted size", dict(shape=(5461, 512, 16, 16, 32, 8, ssa.SSA_BF16), ws_bytes=1024),
     "SSA_E_WORKSPACE"),
    ("one sample past the size limit", dict(shape=(5462, 512, 16, 16, 32, 8, ssa.SSA_BF16)),
     "SSA_E_UNSUPPORTED"),
    ("null x", dict(shape=OK_SHAPE, ptr={"x": 0}), "SSA_E_NULL"),
    ("null out", dict(shape=OK_SHAPE, ptr={"out": 0}), "SSA_E_NULL"),
    # biases are nullable: a NULL bias passes the pointer checks and the call
    # stops at the next rule (a too-small workspace here, so nothing launches)
    ("null v_bias accepted", dict(shape=OK_SHAPE, ptr={"v_bias": 0}, ws_bytes=1024),
     "SSA_E_WORKSPACE"),
    ("all biases null accepted", dict(shape=OK_SHAPE, ptr={"q_bias": 0, "k_bias": 0, "v_bias": 0,
                                                           "out_bias": 0}, ws_bytes=1024),
     "SSA_E_WORKSPACE"),
    ("null norm_weight", dict(shape=OK_SHAPE, ptr={"norm_weight": 0}), "SSA_E_NULL"),
    ("null workspace", dict(shape=OK_SHAPE, ptr={"ws": 0}), "SSA_E_NULL"),
    ("misaligned x", dict(shape=OK_SHAPE, ptr={"x": (1 << 50) + 8}), "SSA_E_ALIGN"),
    ("misaligned weight", dict(shape=OK_SHAPE, ptr={"k_weight": (1 << 50) + 2}), "SSA_E_ALIGN"),
    ("workspace too small", dict(shape=OK_SHAPE, ws_bytes=1024), "SSA_E_WORKSPACE"),
    ("out is x", dict(shape=OK_SHAPE, ptr={"x": 1 << 50, "out": 1 << 50}), "SSA_E_ALIAS"),
    ("out overlaps x", dict(shape=OK_SHAPE, ptr={"x": 1 << 50, "out": (1 << 50) + 256}),
     "SSA_E_ALIAS"),
    ("out overlaps a weight", dict(shape=OK_SHAPE, ptr={"out_weight": 1 << 50,
                                                        "out": (1 << 50) + 4096}), "SSA_E_ALIAS"),
    ("workspace overlaps a bias", dict(shape=OK_SHAPE, ptr={"ws": 1 << 50,
                                                            "q_bias": (1 << 50) + 512}),
     "SSA_E_ALIAS"),
    ("workspace overlaps out", dict(shape=OK_SHAPE, ptr={"ws": 1 << 50, "out": (1 << 50) + 512}),
     "SSA_E_ALIAS"),
])
def test_rejections(case, kw, want):
    assert bnd.STATUS_NAMES[call(**kw)] == want, case
    assert bnd.STATUS_NAMES[call("stage", stage=2, **kw)] == want, case


def test_unknown_stage():
    assert bnd.STATUS_NAMES[call("stage", stage=5, shape=OK_SHAPE)] == "SSA_E_STAGE"
    assert bnd.STATUS_NAMES[call("stage", stage=-1, shape=OK_SHAPE)] == "SSA_E_STAGE"


def test_fused_stage_outside_its_sizes_is_rejected():
    # d = 32: the fused kernel does not cover it; the host says so, nothing launches
    assert bnd.STATUS_NAMES[call("stage", stage=4, shape=OK_SHAPE)] == "SSA_E_UNSUPPORTED"


# Without a GPU the library assumes 256 compute units (the MI355X count), so
# the B * num_heads >= 256 rule reads the same here as on that device.
@pytest.mark.parametrize("shape,want", [
    ((64, 512, 14, 14, 32, 4, ssa.SSA_BF16), True),    # T = 196: 7 key blocks
    ((64, 512, 16, 16, 32, 4, ssa.SSA_BF16), True),    # T = 256: 8 key blocks
    ((22, 1536, 14, 14, 32, 12, ssa.SSA_BF16), True),  # the largest C the LDS table holds
    ((64, 512, 12, 16, 32, 4, ssa.SSA_BF16), False),   # T = 192: 6 blocks, not instantiated
    ((64, 512, 16, 17, 32, 4, ssa.SSA_BF16), False),   # T = 272 > 256
    ((64, 512, 14, 15, 32, 4, ssa.SSA_BF16), False),   # T = 210, not a multiple of 4
    ((63, 512, 14, 14, 32, 4, ssa.SSA_BF16), False),   # 252 (sample, head) pairs < 256 CUs
    ((64, 512, 14, 14, 32, 8, ssa.SSA_BF16), False),   # d = 64
    ((64, 512, 14, 14, 32, 4, ssa.SSA_F32), False),    # fp32
    ((20, 1664, 14, 14, 32, 13, ssa.SSA_BF16), False),  # C past the coefficient table
    ((64, 512, 14, 14, 7, 4, ssa.SSA_BF16), False),    # rejected arguments
    ((0, 512, 14, 14, 32, 4, ssa.SSA_BF16), False),    # empty input
])
def test_uses_fused_stage(shape, want):
    assert ssa.ssa_uses_fused_stage(*shape) is want


@pytest.mark.parametrize("shape", [(0, 64, 8, 8, 8, 2, ssa.SSA_BF16),
                                   (2, 64, 0, 8, 8, 2, ssa.SSA_F32),
                                   (2, 64, 8, 0, 8, 2, ssa.SSA_F32)])
def test_empty_input_is_a_no_op(shape):
    B, C, H, W, G, n, dt = shape
    params = [0] * 10
    st = ssa.ssa_forward(0, 0, params, B, C, H, W, G, n, dt, 0, 0, 0)
    assert st == 0


def test_layout_null_pointer():
    L = ssa.lib()
    assert L.ssa_get_workspace_layout(1, 64, 8, 8, 8, 2, 0, None) == S["SSA_E_NULL"]


def test_python_wrapper_rejects_cpu_tensor():
    import torch
    x = torch.zeros(1, 4, 2, 2)
    p = {k: torch.zeros((4, 4) if k.endswith("weight") and not k.startswith("norm") else (4,))
         for k in bnd.PARAM_ORDER}
    with pytest.raises(ValueError):
        ssa.spatial_self_attention(x, p, 2, 2)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bnd, "_lib", None)
    monkeypatch.setattr(bnd, "LIB_PATH", str(tmp_path / "libssa.so"))
    with pytest.raises(RuntimeError, match="not built"):
        bnd.lib()


# ---------------------------------------------------------------------------
# ssa_forward_ex: the optional steps' rules, all checked before any launch
# ---------------------------------------------------------------------------

def call_ex(shape, opt, ptr=None, ws_bytes=None):
    B, C, H, W, G, n, dt = shape
    fake = Fake()
    p = {k: fake() for k in ["x", "out", "ws"] + list(bnd.PARAM_ORDER)}
    p.update(ptr or {})
    if ws_bytes is None:
        ws_bytes = ssa.ssa_workspace_size(B, C, H, W, G, n, dt) or 1 << 20
    params = [p[k] for k in bnd.PARAM_ORDER]
    return bnd.STATUS_NAMES[ssa.ssa_forward_ex(p["x"], p["out"], params, B, C, H, W, G, n, dt,
                                               opt, p["ws"], ws_bytes, 0)]


def test_ex_query_key_gammas_come_together():
    assert call_ex(OK_SHAPE, bnd.Options(0, 1 << 50, 0, 0)) == "SSA_E_CONSTRAINT"
    assert call_ex(OK_SHAPE, bnd.Options(0, 0, 1 << 50, 0)) == "SSA_E_CONSTRAINT"


def test_ex_rope_needs_even_head():
    assert call_ex((2, 6, 4, 4, 3, 2, ssa.SSA_F32), bnd.Options(0, 0, 0, 1)) == "SSA_E_UNSUPPORTED"


def test_ex_misaligned_option_tensor():
    assert call_ex(OK_SHAPE, bnd.Options((1 << 50) + 2, 0, 0, 0)) == "SSA_E_ALIGN"
    assert call_ex(OK_SHAPE, bnd.Options(0, (1 << 50) + 4, (1 << 51), 0)) == "SSA_E_ALIGN"


def test_ex_option_tensor_must_not_alias_out_or_workspace():
    t = 1 << 50
    # the table of OK_SHAPE is (7*7, 2) bf16 = 196 bytes: out starting inside it overlaps
    assert call_ex(OK_SHAPE, bnd.Options(t, 0, 0, 0), ptr={"out": t + 64}) == "SSA_E_ALIAS"
    assert call_ex(OK_SHAPE, bnd.Options(0, t, t + (1 << 30), 0), ptr={"ws": t + 64}) == "SSA_E_ALIAS"


def test_ex_valid_options_reach_the_workspace_check():
    opt = bnd.Options(1 << 50, 1 << 51, (1 << 51) + (1 << 30), 1)
    assert call_ex(OK_SHAPE, opt, ws_bytes=1024) == "SSA_E_WORKSPACE"
    assert call_ex(OK_SHAPE, None, ws_bytes=1024) == "SSA_E_WORKSPACE"


# ---------------------------------------------------------------------------
# ssa_forward_noalloc: host-side checks (no device call is made on these paths)
# ---------------------------------------------------------------------------

def call_noalloc(shape, ptr=None):
    B, C, H, W, G, n, dt = shape
    fake = Fake()
    p = {k: fake() for k in ["x", "out"] + list(bnd.PARAM_ORDER)}
    p.update(ptr or {})
    st = ssa.ssa_forward_noalloc(p["x"], p["out"], [p[k] for k in bnd.PARAM_ORDER],
                                 B, C, H, W, G, n, dt, 0)
    return bnd.STATUS_NAMES[st]


def test_noalloc_limit_covers_the_workloads():
    from spatial_self_attention_amd.inputs import WORKLOADS
    lim = ssa.ssa_noalloc_max_workspace()
    assert lim == 128 << 20
    for wl in WORKLOADS:
        need = ssa.ssa_workspace_size(wl.B, wl.C, wl.H, wl.W, wl.num_groups, wl.num_heads,
                                      ssa.dtype_code(wl.torch_dtype))
        assert 0 < need <= lim, wl.name


def test_noalloc_rejects_above_its_scratch():
    # 64 x 512 x 64 x 64 bf16: about 1 GB of workspace
    shape = (64, 512, 64, 64, 32, 8, ssa.SSA_BF16)
    assert ssa.ssa_workspace_size(*shape) > ssa.ssa_noalloc_max_workspace()
    assert call_noalloc(shape) == "SSA_E_SCRATCH"


def test_noalloc_validates_before_touching_the_device():
    assert call_noalloc(OK_SHAPE, ptr={"x": 0}) == "SSA_E_NULL"
    assert call_noalloc(OK_SHAPE, ptr={"q_weight": (1 << 44) + 8}) == "SSA_E_ALIGN"
    assert call_noalloc((2, 6, 4, 4, 4, 2, ssa.SSA_BF16)) == "SSA_E_CONSTRAINT"
    assert call_noalloc((2, 64, 4, 4, 8, 2, 7)) == "SSA_E_DTYPE"
    assert call_noalloc((0, 64, 4, 4, 8, 2, ssa.SSA_BF16)) == "SSA_OK"   # empty: nothing to do
