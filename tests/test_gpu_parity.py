"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element.

Bar: max |y_gpu - y_ref| <= 1e-4 (1 + |y_ref|) for fp32 inputs and
<= 2e-2 (1 + |y_ref|) for bf16 inputs with fp32 state.
"""
import os
import sys

import numpy as np
import pytest

import oracle
import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import WORKLOADS, make_inputs, make_random_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
KEYS = ("x", "delta", "A", "B", "C", "D")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup(oracle_lib):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    if not os.path.exists(pkg.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    pkg.load_library()
    pkg.set_spin_limit(0)
    yield


def to_dev(t, dtype):
    dev = torch.device("cuda:0")
    out = []
    for k in KEYS:
        if dtype == "bf16" and k in ("x", "delta", "B", "C"):
            out.append(torch.from_numpy(t[k + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16))
        else:
            out.append(torch.from_numpy(np.ascontiguousarray(t[k])).to(dev))
    return out


def run_gpu(t, dtype, y=None):
    args = to_dev(t, dtype)
    y = pkg.scan_fwd(*args, y=y)
    pkg.sync_check()
    return y


def as_f64(y):
    return y.float().cpu().numpy().astype(np.float64)


def ref_of(t, maps=None):
    return oracle.fwd(*(t[k] for k in KEYS), maps=maps)


def check(got, ref, dtype, what):
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    worst = float(np.max(err)) if err.size else 0.0
    _say(f"  {what}: max |err|/(1+|y|) = {worst:.3e} (bar {TOL[dtype]:.0e})")
    assert np.all(np.isfinite(got)), what
    assert worst <= TOL[dtype], what


@pytest.mark.parametrize("idx", range(len(WORKLOADS)), ids=[w.name for w in WORKLOADS])
def test_workload_full(idx):
    wl = WORKLOADS[idx]
    _say(f"workload {wl.name} {wl}")
    t = make_inputs(wl, seed=0)
    y = as_f64(run_gpu(t, wl.dtype))
    check(y, ref_of(t), wl.dtype, wl.name)


SHAPES = [
    # batch, d_inner, d_state, H, W
    (1, 1, 1, 1, 1), (1, 3, 4, 1, 37), (2, 5, 4, 29, 1), (1, 16, 16, 2, 3),
    (1, 17, 8, 3, 7), (2, 5, 16, 14, 14), (1, 40, 32, 15, 17), (1, 16, 16, 16, 16),
    (1, 7, 12, 63, 65), (1, 33, 16, 64, 80), (1, 16, 5, 129, 3), (1, 9, 64, 17, 9),
    (3, 20, 2, 7, 129), (1, 16, 16, 65, 64),
]


def _seed(shape):
    return sum((i + 1) * v for i, v in enumerate(shape)) % 1000


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("groups", ["4", "8"])
def test_random_shapes(shape, dtype, groups, monkeypatch):
    """Both lane layouts of the strip kernels: 16 channels x 4 state groups
    and 8 x 8 per wave (narrow maps too: the whole-row kernel is off here)."""
    monkeypatch.setenv("SSM2D_GROUPS", groups)
    monkeypatch.setenv("SSM2D_NARROW", "0")
    _say(f"shape {shape} {dtype} groups={groups}")
    t = make_random_inputs(*shape, seed=_seed(shape), dtype=dtype)
    y = as_f64(run_gpu(t, dtype))
    check(y, ref_of(t), dtype, f"{shape} {dtype} groups={groups}")


@pytest.mark.parametrize("groups", ["4", "8"])
@pytest.mark.parametrize("shape", [(2, 16, 16, 19, 64), (1, 24, 8, 7, 40), (1, 8, 4, 9, 16)])
def test_wide_strips(shape, groups, monkeypatch):
    """8-column strips (each lane keeps 8 cells per row)."""
    monkeypatch.setenv("SSM2D_GROUPS", groups)
    monkeypatch.setenv("SSM2D_STRIP", "8")
    _say(f"wide strips {shape} groups={groups}")
    t = make_random_inputs(*shape, seed=_seed(shape))
    check(as_f64(run_gpu(t, "f32")), ref_of(t), "f32", f"K=8 {shape} groups={groups}")


@pytest.mark.parametrize("vec", ["0", "1"])
@pytest.mark.parametrize("strip", ["4", "8"])
@pytest.mark.parametrize("groups", ["4", "8"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_store_forms(vec, strip, groups, dtype, monkeypatch):
    """Both output store forms (one cell per lane, or a channel's cells
    gathered into wider stores; 8-column strips always store cell by cell,
    so there SSM2D_VECSTORE=1 must change nothing) for every strip width,
    lane layout and type, scanning rows left to right and right to left (the
    other directions run 8 groups and 4-column strips). Rows are 4-aligned;
    with 8-column strips the last strip is partial."""
    monkeypatch.setenv("SSM2D_VECSTORE", vec)
    monkeypatch.setenv("SSM2D_STRIP", strip)
    monkeypatch.setenv("SSM2D_GROUPS", groups)
    shape = (2, 24, 16, 11, 44)
    _say(f"store form vec={vec} K={strip} groups={groups} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape), dtype=dtype)
    check(as_f64(run_gpu(t, dtype)), ref_of(t), dtype, f"vec={vec} K={strip} groups={groups}")
    args = to_dev(t, dtype)
    y = pkg.scan_fwd_ex(*args, flags=pkg.FLIP_W)
    pkg.sync_check()
    ref = oracle.fwd(*(t[k] for k in KEYS), flip_w=True)
    check(as_f64(y), ref, dtype, f"flip_w vec={vec} K={strip} groups={groups}")


@pytest.mark.parametrize("groups", ["4", "8"])
@pytest.mark.parametrize("waves", ["1", "2", "3", "8"])
def test_multi_workgroup_chains(waves, groups, monkeypatch):
    """Force short workgroups so strip carries cross workgroups (global path)."""
    monkeypatch.setenv("SSM2D_WAVES", waves)
    monkeypatch.setenv("SSM2D_GROUPS", groups)
    for shape, dtype in (((1, 16, 16, 33, 80), "f32"), ((2, 20, 4, 9, 52), "f32"), ((1, 8, 16, 21, 132), "bf16")):
        _say(f"chains waves={waves} groups={groups} shape {shape} {dtype}")
        t = make_random_inputs(*shape, seed=3, dtype=dtype)
        check(as_f64(run_gpu(t, dtype)), ref_of(t), dtype, f"waves={waves} groups={groups} {shape}")


COOP_SHAPES = [
    # tall maps (H >= 128, W % 4 == 0) cut into several workgroups per chain:
    # the workgroup shares one ring of input rows (cooperative loads)
    ((1, 16, 16, 160, 96), None), ((1, 8, 40, 130, 68), None), ((2, 24, 4, 128, 44), "3"),
    ((1, 16, 16, 131, 64), "8"), ((1, 8, 8, 200, 36), "5"),
]


@pytest.mark.parametrize("case", COOP_SHAPES, ids=[str(c) for c in COOP_SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cooperative_row_ring(case, dtype, monkeypatch):
    shape, waves = case
    monkeypatch.setenv("SSM2D_GROUPS", "8")
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    _say(f"row ring {shape} waves={waves} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape), dtype=dtype)
    check(as_f64(run_gpu(t, dtype)), ref_of(t), dtype, f"row ring {shape} waves={waves}")


def test_special_cases_through_gpu():
    # constant delta (position-independent Abar), A = 0 (Abar = 1), d_state = 0
    t = make_random_inputs(1, 16, 16, 20, 24, seed=5, delta_mode="const")
    check(as_f64(run_gpu(t, "f32")), ref_of(t), "f32", "constant delta")
    t = make_random_inputs(1, 16, 4, 12, 16, seed=6)
    t["A"] = np.zeros_like(t["A"])
    check(as_f64(run_gpu(t, "f32")), ref_of(t), "f32", "A=0 (summed-area)")
    t = make_random_inputs(2, 8, 0, 5, 8, seed=7)
    y = as_f64(run_gpu(t, "f32"))
    ref = (t["D"][None, :, None, None] * t["x"]).astype(np.float64)
    check(y, ref, "f32", "d_state=0")


def test_deterministic_and_every_output_written():
    t = make_inputs(WORKLOADS[1], seed=0)
    args = to_dev(t, "f32")
    y1 = torch.full_like(args[0], float("nan"))
    pkg.scan_fwd(*args, y=y1)
    y2 = torch.full_like(args[0], float("nan"))
    pkg.scan_fwd(*args, y=y2)
    pkg.sync_check()
    assert not torch.isnan(y1).any()
    assert torch.equal(y1, y2)


def test_no_writes_outside_y():
    t = make_random_inputs(2, 17, 16, 13, 21, seed=8)
    args = to_dev(t, "f32")
    n = args[0].numel()
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, device=args[0].device)
    y = buf[guard:guard + n].view(args[0].shape)
    pkg.scan_fwd(*args, y=y)
    pkg.sync_check()
    assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + n:] == 12345.0)
    check(as_f64(y), ref_of(t), "f32", "guarded y")


def test_upper_left_support_bitwise():
    t = make_random_inputs(1, 16, 16, 24, 40, seed=9)
    y0 = as_f64(run_gpu(t, "f32"))
    i0, j0 = 9, 17
    t2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in t.items()}
    t2["x"][:, :, i0, j0] += 1.0
    t2["B"][:, :, i0, j0] += 0.5
    y1 = as_f64(run_gpu(t2, "f32"))
    outside = np.ones((24, 40), dtype=bool)
    outside[i0:, j0:] = False
    assert np.array_equal(y1[:, :, outside], y0[:, :, outside])
    assert not np.array_equal(y1[:, :, i0, j0], y0[:, :, i0, j0])


def test_zero_size_leaves_y_alone():
    x = torch.zeros(1, 4, 0, 8, device="cuda")
    B = torch.zeros(1, 4, 0, 8, device="cuda")
    y = pkg.scan_fwd(x, x, torch.zeros(4, 4, device="cuda"), B, B, torch.zeros(4, device="cuda"))
    assert y.shape == x.shape


def test_timeout_path_reports_and_recovers(monkeypatch):
    """A tiny bound on the kernels' own carry waits: every kernel still exits,
    and a wait that gave up is reported by ssm2d_sync_check."""
    monkeypatch.setenv("SSM2D_WAVES", "1")
    t = make_random_inputs(1, 16, 16, 64, 128, seed=10)
    args = to_dev(t, "f32")
    pkg.set_spin_limit(1)
    try:
        pkg.scan_fwd(*args)
        try:
            pkg.sync_check()
            timed_out = False
        except pkg.Ssm2dError as e:
            assert e.status == pkg.ERR_DEVICE_TIMEOUT
            timed_out = True
        _say(f"  forced wait bound: timed_out={timed_out}")
    finally:
        pkg.set_spin_limit(0)
    pkg.sync_check()  # error word was cleared
    check(as_f64(run_gpu(t, "f32")), ref_of(t), "f32", "after timeout test")
