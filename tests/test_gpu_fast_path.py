"""GPU parity of the two-rows-per-step forward (the plain scan with the
workgroup's shared input row ring: 4 or 8 state groups with 1 or 2 states a
lane, 4-column strips with chains in one or several workgroups, 8-column
strips in one workgroup) against the fp64 oracle, on the shapes that exercise
its edges: the last, partial block of 16 rows and an odd last row; a last
workgroup holding fewer strips; a last 8-column strip half full; padded
states and channels; several batch entries; bottom-to-top rows; bf16. Each
case also runs the general kernel (SSM2D_FAST=0) on the same inputs.

Bars: 1e-4 (1 + |y_ref|) for fp32 inputs, 2e-2 (1 + |y_ref|) for bf16.
"""
import numpy as np
import pytest

import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import make_random_inputs
from test_gpu_parity import KEYS, _say, _setup, as_f64, check, ref_of, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# batch, d_inner, d_state, H, W (W % 4 == 0, H >= 128: the shared row ring)
FAST_SHAPES = [
    (1, 16, 16, 160, 96),    # 24 strips: whole blocks of 16 rows
    (1, 8, 8, 200, 36),      # 1 state a lane; 9 strips (a last workgroup of 1 strip with 8 a group)
    (1, 8, 16, 131, 64),     # odd H: a tail block ending on a single row
    (2, 12, 12, 144, 100),   # padded channels (12 of 16) and states (12 of 16), two batch entries
    (1, 24, 16, 129, 200),   # 50 strips, 2 + 1 chains of channels, H = 8 * 16 + 1
    (1, 8, 5, 150, 124),     # 5 states (1 a lane, 3 padded), 31 strips
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flip_h", [False, True])
@pytest.mark.parametrize("shape", FAST_SHAPES, ids=str)
def test_fast_path(shape, flip_h, dtype, monkeypatch):
    _say(f"fast path {shape} flip_h={flip_h} {dtype}")
    t = make_random_inputs(*shape, seed=sum(shape) + 200 + flip_h, dtype=dtype)
    args = to_dev(t, dtype)
    ref = ref_of(t) if not flip_h else None
    if flip_h:
        import oracle

        ref = oracle.fwd(*(t[k] for k in KEYS), flip_h=True)
    y = pkg.scan_fwd_ex(*args, flip_h=flip_h)
    pkg.sync_check()
    check(as_f64(y), ref, dtype, f"fast {shape} flip_h={flip_h}")
    monkeypatch.setenv("SSM2D_FAST", "0")
    yg = pkg.scan_fwd_ex(*args, flip_h=flip_h)
    pkg.sync_check()
    check(as_f64(yg), ref, dtype, f"general {shape} flip_h={flip_h}")


@pytest.mark.parametrize("waves", ["3", "5", "8"])
def test_fast_path_workgroup_sizes(waves, monkeypatch):
    """Strips per workgroup from 3 to 8 (more couriers, partial last groups)."""
    monkeypatch.setenv("SSM2D_WAVES", waves)
    shape = (1, 16, 16, 140, 120)
    _say(f"fast path waves={waves} {shape}")
    t = make_random_inputs(*shape, seed=230)
    y = pkg.scan_fwd(*to_dev(t, "f32"))
    pkg.sync_check()
    check(as_f64(y), ref_of(t), "f32", f"fast waves={waves}")


def test_fast_path_deterministic_and_guarded():
    """Bitwise equal across runs; cells outside y untouched (guard bands)."""
    shape = (1, 16, 16, 136, 64)
    t = make_random_inputs(*shape, seed=231)
    args = to_dev(t, "f32")
    n = int(np.prod(t["x"].shape))
    buf = torch.full((n + 2048,), 7.0, device="cuda")
    y = buf[1024:1024 + n].view(t["x"].shape)
    pkg.scan_fwd(*args, y=y)
    y1 = y.clone()
    pkg.scan_fwd(*args, y=y)
    pkg.sync_check()
    assert torch.equal(y, y1)
    assert bool((buf[:1024] == 7.0).all()) and bool((buf[1024 + n:] == 7.0).all())
    check(as_f64(y), ref_of(t), "f32", "fast guarded")


# Layouts for many chains (one workgroup a chain; SSM2D_FAST=2): up to
# 16 4-column strips a workgroup (VMamba-like rows of 56 and 60 columns in
# bf16), 8-column strips where 4-column ones do not fit (LDS), 4 state groups
# with 1 and 2 states a lane; and a short map whose chains span workgroups.
LAYOUT_SHAPES = [
    ((32, 64, 16, 20, 56), "bf16"),   # 8 groups, 2 states a lane, 14 4-column strips
    ((32, 64, 16, 19, 60), "bf16"),   # 15 strips, odd H
    ((32, 64, 16, 20, 64), "bf16"),   # 16 4-column strips exceed the LDS: 8-column strips
    ((32, 64, 16, 17, 28), "f32"),    # fp32, 2 states a lane: 7 4-column strips (at most 8 there)
    ((32, 64, 8, 20, 60), "f32"),     # fp32, 1 state a lane, 15 strips exceed the LDS: 8-column, half-full last
    ((32, 64, 8, 13, 48), "f32"),     # fp32, 1 state a lane, 12 4-column strips
    ((32, 64, 8, 18, 56), "f32"),     # 8-column strips, 1 state a lane, fp32
    ((32, 64, 16, 21, 32), "f32"),    # 4-column strips in one workgroup
    ((16, 256, 4, 12, 24), "f32"),    # 4 groups, 1 state a lane
    ((32, 256, 8, 10, 24), "bf16"),   # 4 groups, 2 states a lane
    ((1, 128, 16, 64, 80), "f32"),    # short map, chains across workgroups
]


@pytest.mark.parametrize("case", LAYOUT_SHAPES, ids=str)
def test_fast_path_layouts(case, monkeypatch):
    shape, dtype = case
    _say(f"fast path layout {shape} {dtype}")
    t = make_random_inputs(*shape, seed=sum(shape) + 240, dtype=dtype)
    args = to_dev(t, dtype)
    ref = ref_of(t)
    monkeypatch.setenv("SSM2D_FAST", "2")  # chains in one workgroup too
    assert pkg.fwd_kernels(*shape, bf16=dtype == "bf16") == (1, 0, 0)
    y = pkg.scan_fwd(*args)
    pkg.sync_check()
    check(as_f64(y), ref, dtype, f"fast {shape}")
    monkeypatch.setenv("SSM2D_FAST", "0")
    yg = pkg.scan_fwd(*args)
    pkg.sync_check()
    check(as_f64(yg), ref, dtype, f"general {shape}")


# 8-column strips in chains across workgroups (at most 4 strips and two
# couriers a workgroup): whole and partial last groups, a half-full last
# strip, an odd last row, padded states and channels, bf16, both row orders
WIDE_CHAIN_SHAPES = [
    ((1, 16, 16, 160, 96), "f32", "4"),    # 12 strips: 3 workgroups a chain
    ((1, 32, 16, 131, 200), "f32", "4"),   # 25 strips: a last workgroup of 1 strip, odd H
    ((2, 12, 12, 144, 100), "f32", "3"),   # a half-full last strip, padded channels and states
    ((1, 16, 16, 136, 512), "bf16", "4"),  # giga-pixel width in bf16
    ((1, 8, 8, 150, 64), "f32", "2"),      # 1 state a lane, 2 strips a workgroup
]


@pytest.mark.parametrize("flip_h", [False, True])
@pytest.mark.parametrize("case", WIDE_CHAIN_SHAPES, ids=str)
def test_fast_path_wide_chains(case, flip_h, monkeypatch):
    shape, dtype, waves = case
    monkeypatch.setenv("SSM2D_STRIP", "8")
    monkeypatch.setenv("SSM2D_WAVES", waves)
    assert pkg.fwd_kernels(*shape, bf16=dtype == "bf16") == (1, 0, 0)
    _say(f"fast path, 8-column strips across workgroups {shape} {dtype} waves={waves} flip_h={flip_h}")
    t = make_random_inputs(*shape, seed=sum(shape) + 260 + flip_h, dtype=dtype)
    args = to_dev(t, dtype)
    if flip_h:
        import oracle

        ref = oracle.fwd(*(t[k] for k in KEYS), flip_h=True)
    else:
        ref = ref_of(t)
    y = pkg.scan_fwd_ex(*args, flip_h=flip_h)
    pkg.sync_check()
    check(as_f64(y), ref, dtype, f"fast wide chains {shape}")
    y2 = pkg.scan_fwd_ex(*args, flip_h=flip_h)
    pkg.sync_check()
    assert torch.equal(y, y2)
