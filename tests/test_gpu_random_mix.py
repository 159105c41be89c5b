"""Randomised parity sweep: seeded random shapes, dtypes, directions, orders,
accumulation, gating, step-size options and carried states, each against the
fp64 oracle, so that combinations no hand-picked case names are covered too.
Bars as in the other parity tests."""
import numpy as np
import pytest

import oracle
import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import bf16_bits_from_f32, f32_from_bf16_bits, make_random_inputs
from test_gpu_parity import KEYS, _say, _setup, as_f64, check, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    shape = (int(r.integers(1, 3)), int(r.integers(1, 25)), int(r.choice([0, 1, 3, 4, 8, 12, 16, 32])),
             int(r.integers(1, 40)), int(r.integers(1, 90)))
    dtype = "bf16" if r.random() < 0.4 else "f32"
    kw = dict(flip_h=bool(r.random() < 0.5), flip_w=bool(r.random() < 0.5), vertical_first=bool(r.random() < 0.5))
    opts = dict(gate=bool(r.random() < 0.3), softplus=bool(r.random() < 0.3), carry=bool(r.random() < 0.3),
                waves=str(int(r.integers(1, 4))) if r.random() < 0.3 else None)
    opts["row_carry"] = bool(r.random() < 0.4) and not opts["gate"]  # (carried row states take no gate)
    return shape, dtype, kw, opts


def _dev(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(a)
        return f32_from_bf16_bits(bits).astype(np.float64), torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return a.astype(np.float64), torch.from_numpy(a).cuda()


@pytest.mark.parametrize("seed", range(60))
def test_random_mix(seed, monkeypatch):
    shape, dtype, kw, opts = _case(seed)
    if opts["waves"]:
        monkeypatch.setenv("SSM2D_WAVES", opts["waves"])
    _say(f"mix {seed}: {shape} {dtype} {kw} {opts}")
    t = make_random_inputs(*shape, seed=seed + 500, dtype=dtype)
    r = np.random.default_rng(seed + 600)
    args = to_dev(t, dtype)
    z = zd = None
    if opts["gate"]:
        z, zd = _dev(r.standard_normal(t["x"].shape), dtype)
    raw = t["delta"]
    if opts["softplus"]:
        raw, args[1] = _dev(r.standard_normal(t["x"].shape), dtype)
    b, di, n, H, W = shape
    h0 = r.standard_normal((b, di, n, W)).astype(np.float32) if opts["carry"] else None
    g0 = r.standard_normal((b, di, n, H)).astype(np.float32) if opts["row_carry"] else None
    res = pkg.scan_fwd_mamba(*args, z=zd, delta_softplus=opts["softplus"],
                             h_init=None if h0 is None else torch.from_numpy(h0).cuda(),
                             return_last_state=opts["carry"],
                             hh_init=None if g0 is None else torch.from_numpy(g0).cuda(),
                             return_last_row_state=opts["row_carry"], **kw)
    pkg.sync_check()
    res = res if isinstance(res, tuple) else (res,)
    y = res[0]
    hl = res[1] if opts["carry"] else None
    gl = res[-1] if opts["row_carry"] else None
    # the oracle sees the caller's inputs only: the step size in fp64
    dt = oracle.softplus(raw) if opts["softplus"] else raw
    if opts["carry"] or opts["row_carry"]:
        out = oracle.fwd(t["x"], dt, t["A"], t["B"], t["C"], t["D"], h_init=h0, return_last=opts["carry"],
                         hh_init=g0, return_last_col=opts["row_carry"], **kw)
        out = out if isinstance(out, tuple) else (out,)
        ref = out[0]
        if opts["carry"]:
            check(hl.double().cpu().numpy(), out[1], "f32", f"mix {seed} h_last")
        if opts["row_carry"]:
            check(gl.double().cpu().numpy(), out[-1], "f32", f"mix {seed} hh_last")
    else:
        ref = oracle.fwd(t["x"], dt, t["A"], t["B"], t["C"], t["D"], **kw)
    if z is not None:
        ref = ref * oracle.silu(z)
    check(as_f64(y), ref, dtype, f"mix {seed} y")
