"""GPU parity of the scan-direction, scan-order and multi-direction entry
points (ssm2d_scan_fwd_ex / _ex_bf16) against the fp64 oracle's variants.

The variants follow the pages' own: the vertical-then-horizontal order of the
papernotes.org ablation notes, the reverse scan of its limitations section and
the bidirectional / four-quadrant propagation of the juejin.cn page (part 七,
section 4). Bar as for the forward scan: max |y_gpu - y_ref| <= 1e-4 (1 +
|y_ref|) for fp32 and <= 2e-2 (1 + |y_ref|) for bf16 inputs.
"""
import itertools

import numpy as np
import pytest

import oracle
import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import WORKLOADS, make_inputs, make_random_inputs
from test_gpu_parity import KEYS, _say, _seed, _setup, as_f64, check, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DIRS = list(itertools.product((False, True), repeat=3))  # (flip_h, flip_w, vertical_first)


def _name(d):
    fh, fw, vf = d
    return ("H" if fh else "-") + ("W" if fw else "-") + ("V" if vf else "-")


def run_ex(t, dtype, y=None, D=True, **kw):
    args = to_dev(t, dtype)
    if not D:
        args[5] = None
    y = pkg.scan_fwd_ex(*args, y=y, **kw)
    pkg.sync_check()
    return y


def ref_ex(t, maps=None, D=True, **kw):
    return oracle.fwd(*(t[k] for k in KEYS[:5]), t["D"] if D else None, maps=maps, **kw)


DIR_SHAPES = [
    # batch, d_inner, d_state, H, W: one row, one column, ragged tails (W % 4 = 1, 2, 3),
    # 4-aligned rows over several strips and channel blocks, 64 states, no states
    (1, 3, 4, 1, 37), (2, 5, 4, 29, 1), (1, 17, 8, 13, 7), (1, 9, 16, 14, 30),
    (1, 16, 16, 33, 64), (1, 12, 16, 10, 66), (1, 8, 64, 9, 21), (2, 6, 0, 5, 9),
]


@pytest.mark.parametrize("d", DIRS, ids=_name)
@pytest.mark.parametrize("shape", DIR_SHAPES, ids=[str(s) for s in DIR_SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_directions(shape, d, dtype):
    fh, fw, vf = d
    _say(f"direction {_name(d)} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 7, dtype=dtype)
    y = as_f64(run_ex(t, dtype, flip_h=fh, flip_w=fw, vertical_first=vf))
    check(y, ref_ex(t, flip_h=fh, flip_w=fw, vertical_first=vf), dtype, f"{_name(d)} {shape}")


@pytest.mark.parametrize("d", DIRS, ids=_name)
@pytest.mark.parametrize("waves", ["1", "3"])
def test_directions_multi_workgroup_chains(d, waves, monkeypatch):
    """Strip carries crossing workgroups, in every direction."""
    monkeypatch.setenv("SSM2D_WAVES", waves)
    fh, fw, vf = d
    for shape, dtype in (((1, 16, 16, 33, 80), "f32"), ((1, 8, 16, 21, 130), "bf16")):
        _say(f"chains {_name(d)} waves={waves} {shape} {dtype}")
        t = make_random_inputs(*shape, seed=4, dtype=dtype)
        y = as_f64(run_ex(t, dtype, flip_h=fh, flip_w=fw, vertical_first=vf))
        check(y, ref_ex(t, flip_h=fh, flip_w=fw, vertical_first=vf), dtype, f"{_name(d)} waves={waves} {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [((1, 16, 16, 160, 96), None), ((1, 8, 8, 200, 36), "5")], ids=str)
def test_bottom_to_top_with_shared_row_ring(case, dtype, monkeypatch):
    """Rows bottom to top in the cooperative-load kernels (tall maps)."""
    shape, waves = case
    monkeypatch.setenv("SSM2D_GROUPS", "8")
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    _say(f"bottom to top, row ring {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape), dtype=dtype)
    check(as_f64(run_ex(t, dtype, flip_h=True)), ref_ex(t, flip_h=True), dtype, f"flip_h row ring {shape}")


ACC_FLAGS = [dict(), dict(flip_h=True), dict(flip_w=True, vertical_first=True), dict(flip_h=True, flip_w=True)]


@pytest.mark.parametrize("kw", ACC_FLAGS, ids=str)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 16, 16, 19, 64), (2, 9, 8, 11, 23)], ids=str)
def test_accumulate(shape, dtype, kw):
    """y += result: y starts from seeded values, every cell gets one addition."""
    _say(f"accumulate {kw} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 1, dtype=dtype)
    y0 = np.random.default_rng(5).standard_normal(t["x"].shape).astype(np.float32)
    y = torch.from_numpy(y0).cuda()
    if dtype == "bf16":
        y = y.to(torch.bfloat16)
    start = as_f64(y)
    got = as_f64(run_ex(t, dtype, y=y, accumulate=True, **kw))
    check(got, start + ref_ex(t, **kw), dtype, f"accumulate {kw} {shape}")


@pytest.mark.parametrize("vf", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 16, 16, 21, 44), (2, 5, 4, 9, 13), (1, 8, 16, 1, 30)], ids=str)
def test_four_way(shape, dtype, vf):
    """Sum of the scans from the four corners, skip term once; also without
    a skip term (D = NULL), and accumulated onto itself."""
    _say(f"four-way vf={vf} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 2, dtype=dtype)
    ref = ref_ex(t, four_way=True, vertical_first=vf)
    y = run_ex(t, dtype, four_way=True, vertical_first=vf)
    check(as_f64(y), ref, dtype, f"four-way {shape}")
    check(as_f64(run_ex(t, dtype, D=False, four_way=True, vertical_first=vf)),
          ref_ex(t, D=False, four_way=True, vertical_first=vf), dtype, f"four-way no skip {shape}")
    # accumulated onto itself: y + result, rounded once (bf16: y is the
    # rounded first result, so the reference is that plus the exact sum)
    y1 = as_f64(y)
    y2 = as_f64(run_ex(t, dtype, y=y, four_way=True, vertical_first=vf, accumulate=True))
    check(y2, y1 + ref, dtype, f"four-way accumulated {shape}")


WIDE_SHAPES = [(2, 24, 16, 9, 44), (1, 16, 8, 6, 40), (1, 8, 32, 5, 36)]


@pytest.mark.parametrize("d", DIRS, ids=_name)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=str)
def test_directions_wide_strips(shape, dtype, d, monkeypatch):
    """8-column strips in every direction and order (1, 2 and 4 states a
    lane; the last strip half full where W % 8 == 4), accumulated too."""
    monkeypatch.setenv("SSM2D_STRIP", "8")
    fh, fw, vf = d
    _say(f"wide strips {_name(d)} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 3, dtype=dtype)
    ref = ref_ex(t, flip_h=fh, flip_w=fw, vertical_first=vf)
    y = run_ex(t, dtype, flip_h=fh, flip_w=fw, vertical_first=vf)
    check(as_f64(y), ref, dtype, f"K=8 {_name(d)} {shape}")
    if dtype == "f32":
        y2 = as_f64(run_ex(t, dtype, y=y, accumulate=True, flip_h=fh, flip_w=fw, vertical_first=vf))
        check(y2, 2 * ref, dtype, f"K=8 accumulated {_name(d)} {shape}")


@pytest.mark.parametrize("vf", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_four_way_wide_strips(dtype, vf, monkeypatch):
    monkeypatch.setenv("SSM2D_STRIP", "8")
    shape = WIDE_SHAPES[0]
    _say(f"four-way wide strips vf={vf} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 4, dtype=dtype)
    y = run_ex(t, dtype, four_way=True, vertical_first=vf)
    check(as_f64(y), ref_ex(t, four_way=True, vertical_first=vf), dtype, f"four-way K=8 {shape}")


def test_four_way_deterministic_and_in_bounds():
    t = make_random_inputs(2, 17, 16, 13, 21, seed=8)
    args = to_dev(t, "f32")
    n = args[0].numel()
    guard = 4096
    outs = []
    for _ in range(2):
        buf = torch.full((n + 2 * guard,), 12345.0, device=args[0].device)
        y = buf[guard:guard + n].view(args[0].shape)
        pkg.scan_fwd_ex(*args, y=y, four_way=True)
        pkg.sync_check()
        assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + n:] == 12345.0)
        outs.append(y.clone())
    assert torch.equal(outs[0], outs[1])
    check(as_f64(outs[0]), ref_ex(t, four_way=True), "f32", "four-way guarded")


def test_lower_right_support_bitwise():
    """Scanning from the lower-right corner, a change at (i0, j0) reaches only
    cells above and to the left of it."""
    t = make_random_inputs(1, 16, 16, 24, 40, seed=9)
    kw = dict(flip_h=True, flip_w=True)
    y0 = as_f64(run_ex(t, "f32", **kw))
    i0, j0 = 9, 17
    t2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in t.items()}
    t2["x"][:, :, i0, j0] += 1.0
    y1 = as_f64(run_ex(t2, "f32", **kw))
    outside = np.ones((24, 40), dtype=bool)
    outside[:i0 + 1, :j0 + 1] = False
    assert np.array_equal(y1[:, :, outside], y0[:, :, outside])
    assert not np.array_equal(y1[:, :, i0, j0], y0[:, :, i0, j0])


FULL = [("gigapixel_wsi", dict(four_way=True)), ("vmamba_t_s1", dict(flip_w=True, vertical_first=True)),
        ("wsi_mil", dict(flip_h=True, flip_w=True)), ("grid14", dict(four_way=True, vertical_first=True))]


@pytest.mark.parametrize("case", FULL, ids=lambda c: f"{c[0]}-{c[1]}")
def test_full_size_sampled(case):
    """Full workload sizes, in the launch configuration the benchmark uses;
    sampled maps against the oracle."""
    name, kw = case
    wl = next(w for w in WORKLOADS if w.name == name)
    _say(f"full size {name} {kw}")
    t = make_inputs(wl, seed=0)
    y = as_f64(run_ex(t, wl.dtype, **kw))
    nmaps = wl.batch * wl.d_inner
    maps = np.unique(np.array([0, 1, nmaps // 3, nmaps // 2 + 5, nmaps - 1]))
    ref = ref_ex(t, maps=maps, **kw)
    got = y.reshape(nmaps, wl.H, wl.W)[maps]
    check(got, ref, wl.dtype, f"{name} {kw} maps {maps.tolist()}")


TALL = [((1, 16, 16, 160, 96), None), ((1, 8, 8, 200, 36), "5")]


@pytest.mark.parametrize("d", DIRS, ids=_name)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", TALL, ids=str)
def test_directions_shared_row_ring(case, d, dtype, monkeypatch):
    """Tall maps whose chains span workgroups use the workgroup's shared row
    ring in every direction and order; also accumulated, and four-corner."""
    shape, waves = case
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    fh, fw, vf = d
    kw = dict(flip_h=fh, flip_w=fw, vertical_first=vf)
    _say(f"row ring {_name(d)} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 3, dtype=dtype)
    ref = ref_ex(t, **kw)
    check(as_f64(run_ex(t, dtype, **kw)), ref, dtype, f"row ring {_name(d)} {shape}")
    if dtype == "f32":
        y0 = np.random.default_rng(6).standard_normal(t["x"].shape).astype(np.float32)
        got = as_f64(run_ex(t, dtype, y=torch.from_numpy(y0).cuda(), accumulate=True, **kw))
        check(got, y0 + ref, dtype, f"row ring accumulate {_name(d)} {shape}")
        if not (fh or fw):
            check(as_f64(run_ex(t, dtype, four_way=True, vertical_first=vf)),
                  ref_ex(t, four_way=True, vertical_first=vf), dtype, f"row ring four-way {shape}")


def test_timeout_path_right_to_left(monkeypatch):
    """The bounded carry waits of the right-to-left kernels: a tiny bound
    ends every kernel, is reported, and the next call is exact."""
    monkeypatch.setenv("SSM2D_WAVES", "1")
    t = make_random_inputs(1, 16, 16, 64, 128, seed=36)
    pkg.set_spin_limit(1)
    try:
        run = lambda: pkg.scan_fwd_ex(*to_dev(t, "f32"), flip_w=True, vertical_first=True)
        run()
        try:
            pkg.sync_check()
        except pkg.Ssm2dError as e:
            assert e.status == pkg.ERR_DEVICE_TIMEOUT
    finally:
        pkg.set_spin_limit(0)
    pkg.sync_check()
    check(as_f64(run_ex(t, "f32", flip_w=True, vertical_first=True)),
          ref_ex(t, flip_w=True, vertical_first=True), "f32", "after timeout")


# 4 state groups (16 channels a wave, 4 states a lane) in the direction,
# order, accumulating and gated kernels: used for maps of at most 32 columns,
# an even number of them, 9 to 16 states and many chains (the 14 x 14 grid);
# forced here by the layout hook for small shapes with a ragged channel block,
# rows of 14 (8-byte loads) and of 32 columns (16-byte loads).
G4_SHAPES = [(2, 24, 16, 9, 14), (1, 20, 12, 7, 32)]


@pytest.mark.parametrize("d", DIRS, ids=_name)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", G4_SHAPES, ids=str)
def test_directions_four_groups(shape, dtype, d, monkeypatch):
    monkeypatch.setenv("SSM2D_GROUPS", "4")
    fh, fw, vf = d
    _say(f"4 groups {shape} {_name(d)} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 3, dtype=dtype)
    got = as_f64(run_ex(t, dtype, flip_h=fh, flip_w=fw, vertical_first=vf))
    check(got, ref_ex(t, flip_h=fh, flip_w=fw, vertical_first=vf), dtype, f"4 groups {shape} {_name(d)}")


@pytest.mark.parametrize("vf", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", G4_SHAPES, ids=str)
def test_four_way_four_groups(shape, dtype, vf, monkeypatch):
    monkeypatch.setenv("SSM2D_GROUPS", "4")
    _say(f"4 groups four-way {shape} vf={vf} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 4, dtype=dtype)
    got = as_f64(run_ex(t, dtype, four_way=True, vertical_first=vf))
    check(got, ref_ex(t, four_way=True, vertical_first=vf), dtype, f"4 groups four-way {shape} vf={vf}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", G4_SHAPES, ids=str)
def test_gate_four_groups(shape, dtype, monkeypatch):
    monkeypatch.setenv("SSM2D_GROUPS", "4")
    _say(f"4 groups gate {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 5, dtype=dtype)
    z = np.random.default_rng(_seed(shape) + 6).standard_normal(t["x"].shape).astype(np.float32)
    z_dev = torch.from_numpy(z).cuda()
    if dtype == "bf16":
        z_dev = z_dev.to(torch.bfloat16)
        z = as_f64(z_dev).astype(np.float32)
    for fw, vf in ((False, False), (True, True)):
        y = pkg.scan_fwd_mamba(*to_dev(t, dtype), z=z_dev, flip_w=fw, vertical_first=vf)
        pkg.sync_check()
        ref = oracle.fwd_mamba(*(t[k] for k in KEYS), z=z.astype(np.float64), flip_w=fw, vertical_first=vf)
        check(as_f64(y), ref, dtype, f"4 groups gate {shape} flip_w={fw} vf={vf}")
