"""GPU parity of the Mamba-option entry points (ssm2d_scan_fwd_mamba / _bf16):
step size delta + delta_bias[d] through softplus, and SiLU(z) gating, against
the oracle's fwd_mamba on the same seeded inputs. Bars as for the forward
scan: 1e-4 (1 + |y_ref|) for fp32 and 2e-2 (1 + |y_ref|) for bf16. The oracle
sees only the caller's inputs (fp64 copies of the exact values passed): the
step size, the gate and the four-corner sums are computed in fp64 there."""
import itertools

import numpy as np
import pytest

import oracle
import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import bf16_bits_from_f32, f32_from_bf16_bits, make_random_inputs
from test_gpu_parity import KEYS, _say, _seed, _setup, as_f64, check, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _tensor(a, dtype):
    """Seeded fp32 draws as device tensors, and the exact values the kernel sees."""
    a = np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(a)
        return f32_from_bf16_bits(bits).astype(np.float64), torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return a.astype(np.float64), torch.from_numpy(a).cuda()


SHAPES = [(1, 16, 16, 19, 64), (2, 9, 8, 11, 23), (1, 8, 4, 1, 30), (1, 5, 16, 27, 1)]


@pytest.mark.parametrize("d", list(itertools.product((False, True), repeat=3)), ids=lambda d: "".join("HWV"[i] if v else "-" for i, v in enumerate(d)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
def test_gate(shape, dtype, d):
    fh, fw, vf = d
    _say(f"gate {shape} {dtype} {d}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 21, dtype=dtype)
    z, z_dev = _tensor(np.random.default_rng(_seed(shape)).standard_normal(t["x"].shape) * 2, dtype)
    args = to_dev(t, dtype)
    y = pkg.scan_fwd_mamba(*args, z=z_dev, flip_h=fh, flip_w=fw, vertical_first=vf)
    pkg.sync_check()
    ref = oracle.fwd_mamba(*(t[k] for k in KEYS), z=z, flip_h=fh, flip_w=fw, vertical_first=vf)
    check(as_f64(y), ref, dtype, f"gate {shape} {d}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=str)
@pytest.mark.parametrize("opts", [dict(bias=True, sp=True), dict(bias=False, sp=True), dict(bias=True, sp=False)],
                         ids=str)
def test_step_size(shape, dtype, opts):
    """Raw step sizes of either sign, with the per-channel bias and softplus."""
    _say(f"step size {opts} {shape} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 22, dtype=dtype)
    rng = np.random.default_rng(_seed(shape) + 23)
    raw, raw_dev = _tensor(rng.standard_normal(t["x"].shape) - 0.5, dtype)
    bias = (rng.standard_normal(shape[1]) * 0.5).astype(np.float32) if opts["bias"] else None
    if not opts["sp"]:
        # no softplus: keep the step positive (a negative step makes Abar > 1
        # and the recurrences expanding, outside what the bars are derived for)
        raw, raw_dev = _tensor(np.abs(raw) + 0.05, dtype)
        bias = None if bias is None else np.abs(bias)
    args = to_dev(t, dtype)
    args[1] = raw_dev
    y = pkg.scan_fwd_mamba(*args, delta_bias=None if bias is None else torch.from_numpy(bias).cuda(),
                           delta_softplus=opts["sp"])
    pkg.sync_check()
    ref = oracle.fwd_mamba(t["x"], raw, t["A"], t["B"], t["C"], t["D"], delta_bias=bias, delta_softplus=opts["sp"])
    check(as_f64(y), ref, dtype, f"step size {opts} {shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_everything_together(dtype, monkeypatch):
    """Bias, softplus, gate and the four-corner sum, no skip term; then a
    gated single scan across workgroup chains."""
    shape = (1, 16, 16, 21, 44)
    t = make_random_inputs(*shape, seed=24, dtype=dtype)
    rng = np.random.default_rng(25)
    raw, raw_dev = _tensor(rng.standard_normal(t["x"].shape), dtype)
    z, z_dev = _tensor(rng.standard_normal(t["x"].shape), dtype)
    bias = (rng.standard_normal(shape[1]) * 0.3).astype(np.float32)
    args = to_dev(t, dtype)
    args[1] = raw_dev
    args[5] = None
    y = pkg.scan_fwd_mamba(*args, z=z_dev, delta_bias=torch.from_numpy(bias).cuda(), delta_softplus=True,
                           four_way=True)
    pkg.sync_check()
    ref = oracle.fwd_mamba(t["x"], raw, t["A"], t["B"], t["C"], None, z=z, delta_bias=bias, delta_softplus=True,
                           four_way=True)
    check(as_f64(y), ref, dtype, "everything together")
    monkeypatch.setenv("SSM2D_WAVES", "2")
    shape = (1, 8, 16, 17, 60)
    t = make_random_inputs(*shape, seed=26, dtype=dtype)
    z, z_dev = _tensor(rng.standard_normal(t["x"].shape), dtype)
    y = pkg.scan_fwd_mamba(*to_dev(t, dtype), z=z_dev, flip_w=True)
    pkg.sync_check()
    check(as_f64(y), oracle.fwd_mamba(*(t[k] for k in KEYS), z=z, flip_w=True), dtype, "gated chains")


@pytest.mark.parametrize("d", list(itertools.product((False, True), repeat=3)), ids=lambda d: "".join("HWV"[i] if v else "-" for i, v in enumerate(d)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [((1, 16, 16, 9, 64), None), ((2, 9, 8, 7, 23), None), ((1, 8, 16, 13, 90), "2")],
                         ids=str)
def test_carried_states(case, dtype, d, monkeypatch):
    """A seeded h_init and the returned h_last against the oracle, in every
    direction and order (and across workgroup chains)."""
    shape, waves = case
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    fh, fw, vf = d
    kw = dict(flip_h=fh, flip_w=fw, vertical_first=vf)
    _say(f"carried states {shape} {dtype} {d} waves={waves}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 27, dtype=dtype)
    b, di, n, H, W = shape
    h0 = np.random.default_rng(_seed(shape) + 28).standard_normal((b, di, n, W)).astype(np.float32)
    y, hl = pkg.scan_fwd_mamba(*to_dev(t, dtype), h_init=torch.from_numpy(h0).cuda(), return_last_state=True, **kw)
    pkg.sync_check()
    ref_y, ref_hl = oracle.fwd(*(t[k] for k in KEYS), h_init=h0, return_last=True, **kw)
    check(as_f64(y), ref_y, dtype, f"carried y {shape} {d}")
    check(hl.double().cpu().numpy(), ref_hl, "f32", f"h_last {shape} {d}")


@pytest.mark.parametrize("d", list(itertools.product((False, True), repeat=3)), ids=lambda d: "".join("HWV"[i] if v else "-" for i, v in enumerate(d)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_and_carried_states_wide_strips(dtype, d, monkeypatch):
    """8-column strips (the last one half full): gated output, and a seeded
    h_init with the returned h_last, in every direction and order."""
    monkeypatch.setenv("SSM2D_STRIP", "8")
    fh, fw, vf = d
    kw = dict(flip_h=fh, flip_w=fw, vertical_first=vf)
    shape = (2, 16, 16, 7, 44)
    _say(f"wide strips gate / carried states {d} {dtype}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 31, dtype=dtype)
    rng = np.random.default_rng(_seed(shape) + 32)
    z, z_dev = _tensor(rng.standard_normal(t["x"].shape), dtype)
    y = pkg.scan_fwd_mamba(*to_dev(t, dtype), z=z_dev, **kw)
    pkg.sync_check()
    check(as_f64(y), oracle.fwd_mamba(*(t[k] for k in KEYS), z=z, **kw), dtype, f"K=8 gated {d}")
    b, di, n, H, W = shape
    h0 = rng.standard_normal((b, di, n, W)).astype(np.float32)
    y, hl = pkg.scan_fwd_mamba(*to_dev(t, dtype), h_init=torch.from_numpy(h0).cuda(), return_last_state=True, **kw)
    pkg.sync_check()
    ref_y, ref_hl = oracle.fwd(*(t[k] for k in KEYS), h_init=h0, return_last=True, **kw)
    check(as_f64(y), ref_y, dtype, f"K=8 carried y {d}")
    check(hl.double().cpu().numpy(), ref_hl, "f32", f"K=8 h_last {d}")


@pytest.mark.parametrize("vf", [False, True])
def test_bands_equal_whole_map(vf):
    """Two bands of rows with the carried state in between give the whole
    map's scan (GPU against GPU, and the whole against the oracle)."""
    t = make_random_inputs(1, 16, 16, 40, 64, seed=29)
    args = to_dev(t, "f32")
    y = pkg.scan_fwd_mamba(*args, vertical_first=vf)
    band = lambda a, r: a[:, :, r].contiguous()
    r1, r2 = slice(0, 17), slice(17, 40)
    a1 = [band(args[0], r1), band(args[1], r1), args[2], band(args[3], r1), band(args[4], r1), args[5]]
    a2 = [band(args[0], r2), band(args[1], r2), args[2], band(args[3], r2), band(args[4], r2), args[5]]
    y1, h1 = pkg.scan_fwd_mamba(*a1, vertical_first=vf, return_last_state=True)
    y2 = pkg.scan_fwd_mamba(*a2, vertical_first=vf, h_init=h1)
    pkg.sync_check()
    full = as_f64(y)
    check(full, oracle.fwd(*(t[k] for k in KEYS), vertical_first=vf), "f32", "whole map")
    check(np.concatenate([as_f64(y1), as_f64(y2)], axis=2), full, "f32", "bands vs whole")


@pytest.mark.parametrize("name", ["vmamba_t_s1", "gigapixel_wsi"])
def test_options_full_size_sampled(name):
    """Full workload sizes with bias, softplus and the gate; sampled maps."""
    from selective_state_space_ssm2d_amd.inputs import WORKLOADS, make_inputs

    wl = next(w for w in WORKLOADS if w.name == name)
    dtype = wl.dtype
    t = make_inputs(wl, seed=0)
    rng = np.random.default_rng(30)
    raw, raw_dev = _tensor(rng.standard_normal(t["x"].shape), dtype)
    z, z_dev = _tensor(rng.standard_normal(t["x"].shape), dtype)
    bias = (rng.standard_normal(wl.d_inner) * 0.3).astype(np.float32)
    args = to_dev(t, dtype)
    args[1] = raw_dev
    y = pkg.scan_fwd_mamba(*args, z=z_dev, delta_bias=torch.from_numpy(bias).cuda(), delta_softplus=True)
    pkg.sync_check()
    nmaps = wl.batch * wl.d_inner
    maps = np.unique(np.array([0, 7, nmaps // 2, nmaps - 1]))
    ref = oracle.fwd_mamba(t["x"], raw, t["A"], t["B"], t["C"], t["D"], z=z, delta_bias=bias, delta_softplus=True, maps=maps)
    check(as_f64(y).reshape(nmaps, wl.H, wl.W)[maps], ref, dtype, f"{name} options, maps {maps.tolist()}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_shared_row_ring(dtype):
    """A gated scan of a tall map (the shared row ring), right to left."""
    shape = (1, 16, 16, 160, 96)
    t = make_random_inputs(*shape, seed=31, dtype=dtype)
    z, z_dev = _tensor(np.random.default_rng(31).standard_normal(t["x"].shape), dtype)
    y = pkg.scan_fwd_mamba(*to_dev(t, dtype), z=z_dev, flip_w=True)
    pkg.sync_check()
    check(as_f64(y), oracle.fwd_mamba(*(t[k] for k in KEYS), z=z, flip_w=True), dtype, "gated row ring")


# Carried row states (bands of columns): shapes with several strips and
# channel blocks, ragged rows, chains across workgroups (forced 1- and
# 2-strip workgroups), 8-column strips, one row and one column.
ROW_CARRY_CASES = [((1, 16, 16, 9, 64), None), ((2, 9, 8, 7, 23), None), ((1, 8, 16, 13, 90), "2"),
                   ((1, 16, 16, 6, 40), "1"), ((2, 16, 8, 5, 44), "K8"), ((1, 8, 4, 1, 30), None),
                   ((1, 5, 16, 27, 1), None)]


@pytest.mark.parametrize("d", list(itertools.product((False, True), repeat=3)), ids=lambda d: "".join("HWV"[i] if v else "-" for i, v in enumerate(d)))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ROW_CARRY_CASES, ids=str)
def test_carried_row_states(case, dtype, d, monkeypatch):
    """A seeded hh_init (the row recurrence's state before the first column in
    scan order) and the returned hh_last against the oracle, with h_init /
    h_last too, in every direction and order."""
    shape, opt = case
    if opt == "K8":
        monkeypatch.setenv("SSM2D_STRIP", "8")
    elif opt:
        monkeypatch.setenv("SSM2D_WAVES", opt)
    fh, fw, vf = d
    kw = dict(flip_h=fh, flip_w=fw, vertical_first=vf)
    _say(f"carried row states {shape} {opt} {dtype} {d}")
    t = make_random_inputs(*shape, seed=_seed(shape) + 51, dtype=dtype)
    b, di, n, H, W = shape
    rng = np.random.default_rng(_seed(shape) + 52)
    g0 = rng.standard_normal((b, di, n, H)).astype(np.float32)
    h0 = rng.standard_normal((b, di, n, W)).astype(np.float32)
    y, gl = pkg.scan_fwd_mamba(*to_dev(t, dtype), hh_init=torch.from_numpy(g0).cuda(), return_last_row_state=True,
                               **kw)
    pkg.sync_check()
    ref_y, ref_gl = oracle.fwd(*(t[k] for k in KEYS), hh_init=g0, return_last_col=True, **kw)
    check(as_f64(y), ref_y, dtype, f"row-carried y {shape} {d}")
    check(gl.double().cpu().numpy(), ref_gl, "f32", f"hh_last {shape} {d}")
    y, hl, gl = pkg.scan_fwd_mamba(*to_dev(t, dtype), h_init=torch.from_numpy(h0).cuda(),
                                   hh_init=torch.from_numpy(g0).cuda(), return_last_state=True,
                                   return_last_row_state=True, **kw)
    pkg.sync_check()
    ref_y, ref_hl, ref_gl = oracle.fwd(*(t[k] for k in KEYS), h_init=h0, hh_init=g0, return_last=True,
                                       return_last_col=True, **kw)
    check(as_f64(y), ref_y, dtype, f"tile y {shape} {d}")
    check(hl.double().cpu().numpy(), ref_hl, "f32", f"tile h_last {shape} {d}")
    check(gl.double().cpu().numpy(), ref_gl, "f32", f"tile hh_last {shape} {d}")


@pytest.mark.parametrize("d", list(itertools.product((False, True), repeat=3)), ids=lambda d: "".join("HWV"[i] if v else "-" for i, v in enumerate(d)))
def test_tiles_equal_whole_map(d):
    """A 2 x 2 tiling scanned tile by tile in scan order, each tile taking the
    carries its neighbours handed out, gives the whole map's scan (GPU
    against the oracle), in every direction and order."""
    fh, fw, vf = d
    kw = dict(flip_h=fh, flip_w=fw, vertical_first=vf)
    shape = (1, 16, 16, 37, 70)
    t = make_random_inputs(*shape, seed=53)
    args = to_dev(t, "f32")
    ref = oracle.fwd(*(t[k] for k in KEYS), **kw)
    rows = [slice(0, 15), slice(15, 37)]
    cols = [slice(0, 28), slice(28, 70)]
    if fh:
        rows = rows[::-1]
    if fw:
        cols = cols[::-1]
    tile = lambda a, r, c: a[:, :, r, c].contiguous()
    hcarry, gcarry = {}, {}
    for ri, r in enumerate(rows):
        for ci, c in enumerate(cols):
            a = [tile(args[0], r, c), tile(args[1], r, c), args[2], tile(args[3], r, c), tile(args[4], r, c), args[5]]
            yt, ht, gt = pkg.scan_fwd_mamba(*a, h_init=hcarry.get(ci), hh_init=gcarry.get(ri), return_last_state=True,
                                            return_last_row_state=True, **kw)
            pkg.sync_check()
            hcarry[ci], gcarry[ri] = ht, gt
            check(as_f64(yt), ref[:, :, r, c], "f32", f"tile {ri},{ci} {d}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_carried_row_states_with_step_options(dtype):
    """Carried row states with a step-size bias and softplus (the bf16 call
    then runs the fp32 kernels on widened inputs)."""
    shape = (2, 16, 16, 11, 36)
    t = make_random_inputs(*shape, seed=54, dtype=dtype)
    b, di, n, H, W = shape
    rng = np.random.default_rng(55)
    raw, raw_dev = _tensor(rng.standard_normal(t["x"].shape), dtype)
    bias = rng.standard_normal(di).astype(np.float32) * 0.5
    g0 = rng.standard_normal((b, di, n, H)).astype(np.float32)
    args = to_dev(t, dtype)
    args[1] = raw_dev
    y, gl = pkg.scan_fwd_mamba(*args, delta_bias=torch.from_numpy(bias).cuda(), delta_softplus=True,
                               hh_init=torch.from_numpy(g0).cuda(), return_last_row_state=True, flip_w=True)
    pkg.sync_check()
    dt = oracle.softplus(raw + bias[None, :, None, None].astype(np.float64))
    ref_y, ref_gl = oracle.fwd(t["x"], dt, t["A"], t["B"], t["C"], t["D"], hh_init=g0, return_last_col=True,
                               flip_w=True)
    check(as_f64(y), ref_y, dtype, "row-carried y with step options")
    check(gl.double().cpu().numpy(), ref_gl, "f32", "hh_last with step options")
