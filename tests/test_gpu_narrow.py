"""GPU parity of the whole-row kernel for narrow maps (rows of at most 16
columns, at most 16 states: one wave scans whole rows of 16 channels, no
carry leaves it) against the fp64 oracle: widths 1 to 16 (rows padded to 8
or 16 columns), 0 to 16 states (1, 2 or 4 a lane, padded states), channel
counts that leave a partial block of 16, several batch entries, one row and
many rows, rows bottom to top, no skip term, bf16. Each case also runs the
general kernel (SSM2D_NARROW=0) on the same inputs. Then bitwise
determinism and no writes outside y.

Bars: 1e-4 (1 + |y_ref|) for fp32 inputs, 2e-2 (1 + |y_ref|) for bf16.
"""
import numpy as np
import pytest

import oracle
import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import make_random_inputs
from test_gpu_parity import KEYS, _say, _setup, as_f64, check, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# batch, d_inner, d_state, H, W
SHAPES = [
    (1, 16, 16, 14, 14),   # the 14 x 14 grid, one block of 16 channels
    (2, 20, 16, 9, 13),    # a partial block (4 of 16 channels), two batch entries
    (1, 5, 1, 6, 1),       # one column, one state
    (3, 33, 5, 17, 8),     # 8 columns exactly, 5 states (2 a lane, 3 padded)
    (1, 16, 12, 1, 16),    # one row, 12 states (4 a lane, 4 padded)
    (2, 48, 8, 40, 9),     # 9 columns (padded to 16), 8 states (2 a lane)
    (1, 7, 3, 200, 3),     # many rows, 3 states (1 a lane)
    (4, 64, 16, 30, 16),   # 16 columns exactly, 16 blocks
    (1, 16, 4, 50, 7),     # 4 states: 1 a lane
]


def _seed(shape):
    return sum((i + 3) * v for i, v in enumerate(shape)) % 997


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flip_h", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_narrow_maps(shape, flip_h, dtype, monkeypatch):
    _say(f"narrow {shape} flip_h={flip_h} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + flip_h, dtype=dtype)
    args = to_dev(t, dtype)
    ref = oracle.fwd(*(t[k] for k in KEYS), flip_h=flip_h)
    monkeypatch.setenv("SSM2D_NARROW", "2")
    assert pkg.fwd_kernels(*shape, bf16=dtype == "bf16", flip_h=flip_h) == (0, 0, 1)
    y = pkg.scan_fwd_ex(*args, flip_h=flip_h)
    pkg.sync_check()
    check(as_f64(y), ref, dtype, f"whole rows {shape} flip_h={flip_h}")
    monkeypatch.setenv("SSM2D_NARROW", "0")
    assert pkg.fwd_kernels(*shape, bf16=dtype == "bf16", flip_h=flip_h)[2] == 0
    yg = pkg.scan_fwd_ex(*args, flip_h=flip_h)
    pkg.sync_check()
    check(as_f64(yg), ref, dtype, f"strips {shape} flip_h={flip_h}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_narrow_no_skip_term_and_no_states(dtype, monkeypatch):
    """D = NULL (no skip term), and d_state = 0 (y = D x)."""
    monkeypatch.setenv("SSM2D_NARROW", "2")
    shape = (2, 24, 16, 11, 12)
    t = make_random_inputs(*shape, seed=71, dtype=dtype)
    x, delta, A, B, C, D = to_dev(t, dtype)
    y = pkg.scan_fwd_ex(x, delta, A, B, C, None)
    pkg.sync_check()
    check(as_f64(y), oracle.fwd(*(t[k] for k in KEYS[:5]), None), dtype, "no skip term")
    shape0 = (2, 24, 0, 11, 12)
    t0 = make_random_inputs(*shape0, seed=72, dtype=dtype)
    y0 = pkg.scan_fwd(*to_dev(t0, dtype))
    pkg.sync_check()
    check(as_f64(y0), oracle.fwd(*(t0[k] for k in KEYS)), dtype, "no states: y = D x")


def test_narrow_grid_batch_and_guards():
    """The 14 x 14 grid with 64 x 768 channels (the default plan's choice),
    bitwise equal across runs, cells outside y untouched (guard bands);
    sampled maps against the oracle."""
    shape = (64, 768, 16, 14, 14)
    assert pkg.fwd_kernels(*shape) == (0, 0, 1)
    t = make_random_inputs(*shape, seed=73)
    args = to_dev(t, "f32")
    n = int(np.prod(t["x"].shape))
    buf = torch.full((n + 4096,), 7.0, device="cuda")
    y = buf[2048:2048 + n].view(t["x"].shape)
    pkg.scan_fwd(*args, y=y)
    y1 = y.clone()
    pkg.scan_fwd(*args, y=y)
    pkg.sync_check()
    assert torch.equal(y, y1)
    assert bool((buf[:2048] == 7.0).all()) and bool((buf[2048 + n:] == 7.0).all())
    maps = [0, 767, 768 * 31 + 400, 768 * 64 - 1]
    got = as_f64(y).reshape(-1, 14, 14)[maps]
    check(got, oracle.fwd(*(t[k] for k in KEYS), maps=maps), "f32", "grid batch, sampled maps")
