"""GPU parity of the backward pass (ssm2d_scan_bwd / _bf16) against the fp64
oracle's backward, gradient by gradient, on the same seeded inputs.

Bars. Every gradient: max |g - g_ref| <= tol (1 + |g_ref|), tol = 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs and outputs (fp32 state and arithmetic).
The parameter gradients dA and dD are sums over every cell of the batch: the
kernels sum each row's terms in fp32 and the row sums in fp64, so their
rounding does not grow with the number of cells and the same bar holds.
"""
import itertools

import numpy as np
import pytest

import oracle
import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import (WORKLOADS, bf16_bits_from_f32, f32_from_bf16_bits,
                                                    make_inputs, make_random_inputs)
from test_gpu_parity import KEYS, _say, _seed, _setup, as_f64, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dx", "ddelta", "dA", "dB", "dC", "dD")


def make_dy(t, dtype, seed):
    """Seeded upstream gradient with the shape of y; for bf16 the exact bf16
    values (the oracle sees what the kernel sees)."""
    dy = np.random.default_rng(seed).standard_normal(t["x"].shape).astype(np.float32)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(dy)
        return f32_from_bf16_bits(bits), torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return dy, torch.from_numpy(dy).cuda()


def run_bwd(t, dtype, dy_dev):
    args = to_dev(t, dtype)
    g = pkg.scan_bwd(*args, dy_dev)
    pkg.sync_check()
    return {k: as_f64(v) for k, v in g.items()}


def check_grads(got, ref, dtype, cells, what):
    for k in NAMES:
        tol = TOL[dtype]
        g, r = got[k], ref[k]
        assert g.shape == r.shape, (k, g.shape, r.shape)
        if g.size == 0:
            continue
        err = float(np.max(np.abs(g - r) / (1.0 + np.abs(r))))
        _say(f"  {what} {k}: max |err|/(1+|g|) = {err:.3e} (bar {tol:.1e})")
        assert np.all(np.isfinite(g)), (what, k)
        assert err <= tol, (what, k)


BWD_SHAPES = [
    # batch, d_inner, d_state, H, W: one cell, one row, one column, ragged
    # tails (W % 4 = 1, 2, 3), several strips / channel blocks / batch entries,
    # 32 states, odd state counts
    (1, 1, 1, 1, 1), (1, 3, 4, 1, 37), (2, 5, 4, 29, 1), (1, 17, 8, 13, 7),
    (1, 9, 16, 14, 30), (2, 16, 16, 21, 64), (1, 12, 16, 10, 66), (1, 8, 32, 9, 21),
    (3, 20, 3, 7, 45), (1, 24, 5, 33, 19),
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=[str(s) for s in BWD_SHAPES])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward(shape, dtype):
    _say(f"backward {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 11, dtype=dtype)
    dy, dy_dev = make_dy(t, dtype, _seed(shape) + 12)
    got = run_bwd(t, dtype, dy_dev)
    ref = oracle.bwd(*(t[k] for k in KEYS), dy)
    check_grads(got, ref, dtype, shape[0] * shape[3] * shape[4], f"{shape} {dtype}")


@pytest.mark.parametrize("waves", ["1", "2", "3"])
def test_backward_multi_workgroup_chains(waves, monkeypatch):
    """Adjoint carries crossing workgroups (right to left)."""
    monkeypatch.setenv("SSM2D_WAVES", waves)
    for shape, dtype in (((1, 16, 16, 33, 80), "f32"), ((1, 8, 16, 21, 130), "bf16")):
        _say(f"backward chains waves={waves} {shape} {dtype}")
        t = make_random_inputs(*shape, seed=5, dtype=dtype)
        dy, dy_dev = make_dy(t, dtype, 6)
        got = run_bwd(t, dtype, dy_dev)
        check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), dtype, shape[0] * shape[3] * shape[4],
                    f"waves={waves} {shape}")


def test_backward_special_cases():
    # no states: dx = dy D, dD = sum dy x; empty maps: dA, dD zeroed
    t = make_random_inputs(2, 8, 0, 5, 8, seed=7)
    dy, dy_dev = make_dy(t, "f32", 8)
    got = run_bwd(t, "f32", dy_dev)
    check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), "f32", 80, "d_state=0")
    x = torch.zeros(1, 4, 0, 8, device="cuda")
    B = torch.zeros(1, 3, 0, 8, device="cuda")
    out = {"dA": torch.full((4, 3), 7.0, device="cuda"), "dD": torch.full((4,), 7.0, device="cuda")}
    g = pkg.scan_bwd(x, x, torch.zeros(4, 3, device="cuda"), B, B, torch.zeros(4, device="cuda"), x, out=out)
    torch.cuda.synchronize()
    assert torch.all(g["dA"] == 0) and torch.all(g["dD"] == 0)


def test_backward_repeated_calls_and_shape_changes():
    """The workspace is reused and regrown; a smaller ragged call after a larger
    one (stale pad columns) is still exact to the bar."""
    for shape in ((1, 16, 16, 19, 64), (1, 9, 8, 17, 13), (1, 16, 16, 19, 64)):
        t = make_random_inputs(*shape, seed=_seed(shape))
        dy, dy_dev = make_dy(t, "f32", 9)
        got = run_bwd(t, "f32", dy_dev)
        check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), "f32", shape[3] * shape[4], f"repeat {shape}")


def test_backward_full_wsi_mil():
    """The WSI-MIL workload at full size (every gradient element)."""
    wl = next(w for w in WORKLOADS if w.name == "wsi_mil")
    t = make_inputs(wl, seed=0)
    dy, dy_dev = make_dy(t, wl.dtype, 10)
    got = run_bwd(t, wl.dtype, dy_dev)
    check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), wl.dtype, wl.batch * wl.H * wl.W, "wsi_mil")


@pytest.mark.parametrize("name", ["vmamba_t_s1", "grid14", "gigapixel_wsi"])
def test_backward_full_workloads(name):
    """The other workloads at full size, in the launch configuration the
    benchmark times: every gradient element against the oracle."""
    wl = next(w for w in WORKLOADS if w.name == name)
    _say(f"backward full size {name}")
    t = make_inputs(wl, seed=0)
    dy, dy_dev = make_dy(t, wl.dtype, 13)
    got = run_bwd(t, wl.dtype, dy_dev)
    check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), wl.dtype, wl.batch * wl.H * wl.W, name)


@pytest.mark.parametrize("shape", [(1, 16, 16, 160, 96), (1, 8, 4, 140, 48), (1, 8, 32, 130, 64)], ids=str)
def test_backward_tall_map(shape):
    """Tall maps (1, 2 and 4 states a lane): the stored-state pass and the
    adjoint pass use the shared row ring."""
    t = make_random_inputs(*shape, seed=32)
    dy, dy_dev = make_dy(t, "f32", 33)
    got = run_bwd(t, "f32", dy_dev)
    check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), "f32", shape[3] * shape[4], f"tall map {shape}")


def test_backward_timeout_path_reports_and_recovers(monkeypatch):
    """A tiny bound on the kernels' own carry waits: the three backward
    kernels still exit, the error word reports the timeout, and the next
    call is exact again."""
    monkeypatch.setenv("SSM2D_WAVES", "1")
    t = make_random_inputs(1, 16, 16, 64, 128, seed=34)
    dy, dy_dev = make_dy(t, "f32", 35)
    args = to_dev(t, "f32")
    pkg.set_spin_limit(1)
    try:
        pkg.scan_bwd(*args, dy_dev)
        try:
            pkg.sync_check()
            timed_out = False
        except pkg.Ssm2dError as e:
            assert e.status == pkg.ERR_DEVICE_TIMEOUT
            timed_out = True
        _say(f"  forced wait bound (backward): timed_out={timed_out}")
    finally:
        pkg.set_spin_limit(0)
    pkg.sync_check()
    got = run_bwd(t, "f32", dy_dev)
    check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), "f32", 64 * 128, "after timeout")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("opts", [dict(gate=True, bias=True, sp=True), dict(gate=True, bias=False, sp=False),
                                  dict(gate=False, bias=True, sp=True), dict(gate=False, bias=False, sp=True)],
                         ids=str)
def test_backward_mamba_options(opts, dtype):
    """Gradients of the gated scan with the step-size bias and softplus,
    including dz and d bias, against the oracle's chain rule (itself pinned by
    finite differences)."""
    from selective_state_space_ssm2d_amd.inputs import bf16_bits_from_f32, f32_from_bf16_bits

    shape = (2, 12, 16, 17, 30)
    t = make_random_inputs(*shape, seed=38, dtype=dtype)
    r = np.random.default_rng(38)

    def dev(a):
        a = np.asarray(a, dtype=np.float32)
        if dtype == "bf16":
            bits = bf16_bits_from_f32(a)
            return f32_from_bf16_bits(bits).astype(np.float64), torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        return a.astype(np.float64), torch.from_numpy(a).cuda()

    raw, raw_dev = dev(r.standard_normal(t["x"].shape) - 0.2) if opts["sp"] else dev(np.abs(r.standard_normal(t["x"].shape)) + 0.1)
    z, z_dev = dev(r.standard_normal(t["x"].shape)) if opts["gate"] else (None, None)
    bias = (np.abs(r.standard_normal(shape[1])) * 0.3).astype(np.float32) if opts["bias"] else None
    dy, dy_dev = make_dy(t, dtype, 39)
    args = to_dev(t, dtype)
    args[1] = raw_dev
    g = pkg.scan_bwd_mamba(*args, dy_dev, z=z_dev, delta_bias=None if bias is None else torch.from_numpy(bias).cuda(),
                           delta_softplus=opts["sp"])
    pkg.sync_check()
    got = {k: v.double().cpu().numpy() for k, v in g.items()}
    # the oracle takes only the caller's inputs; every intermediate is fp64
    ref = oracle.bwd_mamba(t["x"], raw, t["A"], t["B"], t["C"], t["D"], dy, z=z, delta_bias=bias,
                           delta_softplus=opts["sp"])
    cells = shape[0] * shape[3] * shape[4]
    check_grads(got, ref, dtype, cells, f"options {opts}")
    if "dz" in ref:
        err = float(np.max(np.abs(got["dz"] - ref["dz"]) / (1.0 + np.abs(ref["dz"]))))
        _say(f"  options {opts} dz: {err:.3e} (bar {TOL[dtype]:.1e})")
        assert err <= TOL[dtype], "dz"
    if "ddelta_bias" in ref:
        # d bias[d] sums d delta over the channel's cells: its bar is the sum
        # of the elementwise bars of those d delta values
        bar = TOL[dtype] * np.sum(1.0 + np.abs(ref["ddelta"]), axis=(0, 2, 3))
        worst = float(np.max(np.abs(got["ddelta_bias"] - ref["ddelta_bias"]) / bar))
        _say(f"  options {opts} ddelta_bias: {worst:.3e} of the summed bar")
        assert worst <= 1.0, "ddelta_bias"


FLIPS = [(True, False), (False, True), (True, True)]


@pytest.mark.parametrize("fl", FLIPS, ids=lambda f: ("H" if f[0] else "-") + ("W" if f[1] else "-"))
@pytest.mark.parametrize("shape", [(1, 3, 4, 1, 37), (2, 5, 4, 29, 1), (1, 17, 8, 13, 7), (1, 9, 16, 14, 30),
                                   (2, 16, 16, 21, 64), (1, 8, 32, 9, 21)], ids=str)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_other_directions(shape, fl, dtype):
    """The backward of the scans from the other corners (ssm2d_scan_bwd_ex)."""
    fh, fw = fl
    _say(f"backward flips {fl} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 40, dtype=dtype)
    dy, dy_dev = make_dy(t, dtype, _seed(shape) + 41)
    g = pkg.scan_bwd(*to_dev(t, dtype), dy_dev, flip_h=fh, flip_w=fw)
    pkg.sync_check()
    got = {k: as_f64(v) for k, v in g.items()}
    ref = oracle.bwd(*(t[k] for k in KEYS), dy, flip_h=fh, flip_w=fw)
    check_grads(got, ref, dtype, shape[0] * shape[3] * shape[4], f"flips {fl} {shape}")


@pytest.mark.parametrize("fl", FLIPS, ids=lambda f: ("H" if f[0] else "-") + ("W" if f[1] else "-"))
@pytest.mark.parametrize("case", [((1, 16, 16, 33, 80), "1", "f32"), ((1, 8, 16, 21, 130), "3", "bf16"),
                                  ((1, 16, 16, 160, 96), None, "f32"), ((1, 8, 16, 150, 64), None, "bf16"),
                                  ((1, 8, 4, 140, 48), None, "f32"), ((1, 8, 32, 130, 64), None, "f32")],
                         ids=str)
def test_backward_other_directions_chains(case, fl, monkeypatch):
    """Other corners with chains across workgroups, and tall maps (the
    stored-state pass and the adjoint pass both use the shared row ring)."""
    shape, waves, dtype = case
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    fh, fw = fl
    t = make_random_inputs(*shape, seed=43, dtype=dtype)
    dy, dy_dev = make_dy(t, dtype, 44)
    g = pkg.scan_bwd(*to_dev(t, dtype), dy_dev, flip_h=fh, flip_w=fw)
    pkg.sync_check()
    got = {k: as_f64(v) for k, v in g.items()}
    check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy, flip_h=fh, flip_w=fw), dtype,
                shape[0] * shape[3] * shape[4], f"flips {fl} chains {case}")


DIRS4 = [(False, False), (True, False), (False, True), (True, True)]


@pytest.mark.parametrize("fl", DIRS4, ids=lambda f: "V" + ("H" if f[0] else "-") + ("W" if f[1] else "-"))
@pytest.mark.parametrize("shape", [(1, 3, 4, 1, 37), (2, 5, 4, 29, 1), (1, 17, 8, 13, 7), (1, 9, 16, 14, 30),
                                   (2, 16, 16, 21, 64), (1, 8, 32, 9, 21), (1, 8, 16, 70, 150)], ids=str)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_vertical_first(shape, fl, dtype):
    """The backward of the vertical-first order in every direction
    (ssm2d_scan_bwd_ex with SSM2D_VERTICAL_FIRST): non-square maps, ragged
    sides, one row, one column, maps wider than a transpose tile."""
    fh, fw = fl
    _say(f"backward vertical-first flips {fl} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 45, dtype=dtype)
    dy, dy_dev = make_dy(t, dtype, _seed(shape) + 46)
    g = pkg.scan_bwd(*to_dev(t, dtype), dy_dev, flip_h=fh, flip_w=fw, vertical_first=True)
    pkg.sync_check()
    got = {k: as_f64(v) for k, v in g.items()}
    ref = oracle.bwd(*(t[k] for k in KEYS), dy, flip_h=fh, flip_w=fw, vertical_first=True)
    check_grads(got, ref, dtype, shape[0] * shape[3] * shape[4], f"vertical-first {fl} {shape}")


def test_backward_vertical_first_full_vmamba():
    """VMamba stage 1 (bf16) at full size, vertical-first order: every
    gradient element against the oracle."""
    wl = next(w for w in WORKLOADS if w.name == "vmamba_t_s1")
    t = make_inputs(wl, seed=0)
    dy, dy_dev = make_dy(t, wl.dtype, 47)
    g = pkg.scan_bwd(*to_dev(t, wl.dtype), dy_dev, vertical_first=True)
    pkg.sync_check()
    got = {k: as_f64(v) for k, v in g.items()}
    check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy, vertical_first=True), wl.dtype,
                wl.batch * wl.H * wl.W, "vmamba vertical-first")


# Carried vertical states (bands of rows): the forward started from h_init,
# the loss also takes dh_last through h_last. Shapes: several strips and
# channel blocks, ragged rows (W % 4 = 1, 3), one row, one column, chains
# across workgroups (forced 1-strip workgroups: the courier-free adjoint),
# and a tall map with the shared row ring.
CARRY_CASES = [((1, 16, 16, 9, 64), None), ((2, 9, 8, 7, 23), None), ((1, 8, 16, 1, 29), None),
               ((1, 5, 16, 27, 1), None), ((1, 16, 16, 13, 40), "1"), ((1, 16, 16, 140, 96), None)]


@pytest.mark.parametrize("flips", [(False, False), (True, False), (False, True), (True, True)],
                         ids=lambda f: "".join("HW"[i] if v else "-" for i, v in enumerate(f)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CARRY_CASES, ids=str)
def test_carried_state_backward(case, dtype, flips, monkeypatch):
    shape, waves = case
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    fh, fw = flips
    _say(f"carried-state backward {shape} {dtype} flips={flips} waves={waves}")
    t = make_random_inputs(*shape, seed=sum(shape) + 61, dtype=dtype)
    b, di, n, H, W = shape
    r = np.random.default_rng(sum(shape) + 62)
    h0 = r.standard_normal((b, di, n, W)).astype(np.float32)
    gl = r.standard_normal((b, di, n, W)).astype(np.float32)
    dy, dy_dev = make_dy(t, dtype, sum(shape) + 63)
    g = pkg.scan_bwd_mamba(*to_dev(t, dtype), dy_dev, h_init=torch.from_numpy(h0).cuda(),
                           dh_last=torch.from_numpy(gl).cuda(), flip_h=fh, flip_w=fw)
    pkg.sync_check()
    got = {k: v.double().cpu().numpy() for k, v in g.items()}
    ref = oracle.bwd(*(t[k] for k in ("x", "delta", "A", "B", "C", "D")), dy, h_init=h0, dh_last=gl, flip_h=fh,
                     flip_w=fw)
    check_grads(got, ref, dtype, b * H * W, f"carried {shape} {flips}")
    err = float(np.max(np.abs(got["dh_init"] - ref["dh_init"]) / (1.0 + np.abs(ref["dh_init"]))))
    _say(f"  dh_init: {err:.3e}")
    assert err <= TOL["f32"] * max(1.0, np.sqrt(H / 64.0)), "dh_init"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_carried_state_backward_with_options(dtype):
    """Carried states with the gate, a step-size bias and softplus, scanned
    from the lower-right corner."""
    shape = (2, 12, 16, 11, 30)
    t = make_random_inputs(*shape, seed=64, dtype=dtype)
    b, di, n, H, W = shape
    r = np.random.default_rng(64)

    def dev(a):
        a = np.asarray(a, dtype=np.float32)
        if dtype == "bf16":
            bits = bf16_bits_from_f32(a)
            return f32_from_bf16_bits(bits).astype(np.float64), torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        return a.astype(np.float64), torch.from_numpy(a).cuda()

    raw, raw_dev = dev(r.standard_normal(t["x"].shape) - 0.2)
    z, z_dev = dev(r.standard_normal(t["x"].shape))
    bias = (np.abs(r.standard_normal(di)) * 0.3).astype(np.float32)
    h0 = r.standard_normal((b, di, n, W)).astype(np.float32)
    gl = r.standard_normal((b, di, n, W)).astype(np.float32)
    dy, dy_dev = make_dy(t, dtype, 65)
    args = to_dev(t, dtype)
    args[1] = raw_dev
    g = pkg.scan_bwd_mamba(*args, dy_dev, z=z_dev, delta_bias=torch.from_numpy(bias).cuda(), delta_softplus=True,
                           h_init=torch.from_numpy(h0).cuda(), dh_last=torch.from_numpy(gl).cuda(), flip_h=True,
                           flip_w=True)
    pkg.sync_check()
    got = {k: v.double().cpu().numpy() for k, v in g.items()}
    ref = oracle.bwd_mamba(t["x"], raw, t["A"], t["B"], t["C"], t["D"], dy, z=z, delta_bias=bias,
                           delta_softplus=True, h_init=h0, dh_last=gl, flip_h=True, flip_w=True)
    check_grads(got, ref, dtype, b * H * W, "carried with options")
    for k in ("dz", "dh_init"):
        err = float(np.max(np.abs(got[k] - ref[k]) / (1.0 + np.abs(ref[k]))))
        _say(f"  {k}: {err:.3e}")
        assert err <= TOL[dtype if k == "dz" else "f32"], k


TILE_CASES = [((1, 16, 16, 9, 64), None), ((2, 9, 8, 7, 23), None), ((1, 8, 16, 1, 29), None),
              ((1, 5, 16, 27, 1), None), ((1, 16, 16, 13, 40), "1"), ((1, 16, 16, 140, 96), None)]


@pytest.mark.parametrize("d", list(itertools.product((False, True), repeat=3)),
                         ids=lambda d: "".join("HWV"[i] if v else "-" for i, v in enumerate(d)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", TILE_CASES, ids=str)
def test_tile_backward(case, dtype, d, monkeypatch):
    """The backward of a tile: both carried states in, dL/d(both last states)
    in, every gradient plus dL/dh_init and dL/dhh_init out, against the
    oracle in every direction and order."""
    shape, waves = case
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    fh, fw, vf = d
    kw = dict(flip_h=fh, flip_w=fw, vertical_first=vf)
    _say(f"tile backward {shape} {dtype} {d} waves={waves}")
    t = make_random_inputs(*shape, seed=sum(shape) + 71, dtype=dtype)
    b, di, n, H, W = shape
    r = np.random.default_rng(sum(shape) + 72)
    h0 = r.standard_normal((b, di, n, W)).astype(np.float32)
    gl = r.standard_normal((b, di, n, W)).astype(np.float32)
    g0 = r.standard_normal((b, di, n, H)).astype(np.float32)
    ggl = r.standard_normal((b, di, n, H)).astype(np.float32)
    dy, dy_dev = make_dy(t, dtype, sum(shape) + 73)
    cu = lambda a: torch.from_numpy(a).cuda()
    g = pkg.scan_bwd_mamba(*to_dev(t, dtype), dy_dev, h_init=cu(h0), dh_last=cu(gl), hh_init=cu(g0),
                           dhh_last=cu(ggl), **kw)
    pkg.sync_check()
    got = {k: v.double().cpu().numpy() for k, v in g.items()}
    ref = oracle.bwd(*(t[k] for k in ("x", "delta", "A", "B", "C", "D")), dy, h_init=h0, dh_last=gl, hh_init=g0,
                     dhh_last=ggl, **kw)
    check_grads(got, ref, dtype, b * H * W, f"tile {shape} {d}")
    for k, length in (("dh_init", H), ("dhh_init", W)):
        err = float(np.max(np.abs(got[k] - ref[k]) / (1.0 + np.abs(ref[k])))) if ref[k].size else 0.0
        _say(f"  {k}: {err:.3e}")
        assert err <= TOL["f32"] * max(1.0, np.sqrt(max(H, W) / 64.0)), k


@pytest.mark.parametrize("d", [(False, False, False), (True, True, False), (False, True, True)],
                         ids=lambda d: "".join("HWV"[i] if v else "-" for i, v in enumerate(d)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 9, 40, 7, 23), (2, 8, 64, 13, 40), (1, 16, 33, 5, 64)], ids=str)
def test_many_states_backward(shape, dtype, d):
    """More states than the backward's kernels hold (32): chunks of states,
    their dx and d delta summed; plain, and with both carried states."""
    fh, fw, vf = d
    kw = dict(flip_h=fh, flip_w=fw, vertical_first=vf)
    _say(f"many-state backward {shape} {dtype} {d}")
    t = make_random_inputs(*shape, seed=sum(shape) + 81, dtype=dtype)
    b, di, n, H, W = shape
    dy, dy_dev = make_dy(t, dtype, sum(shape) + 82)
    keys = ("x", "delta", "A", "B", "C", "D")
    if not any(d):
        got = run_bwd(t, dtype, dy_dev)
        check_grads(got, oracle.bwd(*(t[k] for k in keys), dy), dtype, b * H * W, f"{n} states {shape}")
    r = np.random.default_rng(sum(shape) + 83)
    h0, gl = (r.standard_normal((b, di, n, W)).astype(np.float32) for _ in range(2))
    g0, ggl = (r.standard_normal((b, di, n, H)).astype(np.float32) for _ in range(2))
    cu = lambda a: torch.from_numpy(a).cuda()
    g = pkg.scan_bwd_mamba(*to_dev(t, dtype), dy_dev, h_init=cu(h0), dh_last=cu(gl), hh_init=cu(g0),
                           dhh_last=cu(ggl), **kw)
    pkg.sync_check()
    got = {k: v.double().cpu().numpy() for k, v in g.items()}
    ref = oracle.bwd(*(t[k] for k in keys), dy, h_init=h0, dh_last=gl, hh_init=g0, dhh_last=ggl, **kw)
    check_grads(got, ref, dtype, b * H * W, f"{n} states, carried {shape} {d}")
    for k in ("dh_init", "dhh_init"):
        err = float(np.max(np.abs(got[k] - ref[k]) / (1.0 + np.abs(ref[k]))))
        _say(f"  {k}: {err:.3e}")
        assert err <= TOL["f32"] * max(1.0, np.sqrt(max(H, W) / 64.0)), k
