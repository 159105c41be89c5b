"""GPU tests of the library's launch machinery around the scan: HIP-graph
capture and replay, the carry-tag epoch and its wrap, timeouts that surface on
the next call, the release of workspaces, launches that share the GPU with
each other, the carry ring's overflow rows and the bounded ring's blocks of
tickets.

The carry words that link the tiles of one map across workgroups are tagged
with an epoch kept in device memory; every launch (every replay of a captured
one too) advances it, and its wrap clears the ring. Parity bars as for the
forward scan and its backward (1e-4 (1 + |ref|) in fp32).
"""
import numpy as np
import pytest

import oracle
import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import make_random_inputs
from test_gpu_backward import NAMES, check_grads, make_dy
from test_gpu_parity import KEYS, _say, _setup, as_f64, check, ref_of, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# chains cut into several workgroups: the giga-pixel layout (the bounded
# carry ring with overflow rows, or a slot a row) and forced one-strip
# workgroups (couriers on every boundary)
CHAIN_CASES = [((1, 32, 16, 96, 512), None, None), ((1, 32, 16, 96, 512), None, "0"), ((1, 16, 16, 40, 96), "1", None)]


def _copy_inputs(dst, t):
    for d, s in zip(dst, to_dev(t, "f32")):
        d.copy_(s)


@pytest.mark.parametrize("case", CHAIN_CASES, ids=str)
def test_graph_replays_forward(case, monkeypatch):
    """A forward captured in a HIP graph and replayed with new inputs copied
    in before each replay, with eager calls on the same stream in between:
    every replay and every eager call matches the oracle."""
    shape, waves, ring = case
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    if ring:
        monkeypatch.setenv("SSM2D_RING", ring)
    s = torch.cuda.Stream()
    t0 = make_random_inputs(*shape, seed=60)
    with torch.cuda.stream(s):
        args = to_dev(t0, "f32")
        y = pkg.scan_fwd(*args)  # warm-up: the stream's workspace exists before the capture
    s.synchronize()
    check(as_f64(y), ref_of(t0), "f32", f"warm-up {shape}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pkg.scan_fwd(*args, y=y)
    for r in range(3):
        t = make_random_inputs(*shape, seed=61 + r)
        with torch.cuda.stream(s):
            _copy_inputs(args, t)
            y.fill_(float("nan"))
        g.replay()
        s.synchronize()
        _say(f"  replay {r}")
        check(as_f64(y), ref_of(t), "f32", f"graph replay {r} {shape}")
        # an eager call between replays (it advances the same epoch)
        te = make_random_inputs(*shape, seed=70 + r)
        with torch.cuda.stream(s):
            ae = to_dev(te, "f32")
            ye = pkg.scan_fwd(*ae)
        s.synchronize()
        check(as_f64(ye), ref_of(te), "f32", f"eager between replays {r}")
    pkg.sync_check(s)


def test_graph_replays_backward(monkeypatch):
    """The backward (stored-state pass, adjoint pass with chains across
    workgroups, channel sums) captured and replayed with new inputs."""
    monkeypatch.setenv("SSM2D_WAVES", "2")
    shape = (1, 16, 16, 24, 72)
    s = torch.cuda.Stream()
    t0 = make_random_inputs(*shape, seed=80)
    dy0, _ = make_dy(t0, "f32", 81)
    with torch.cuda.stream(s):
        args = to_dev(t0, "f32")
        dy_dev = torch.from_numpy(np.asarray(dy0, dtype=np.float32)).cuda()
        out = pkg.scan_bwd(*args, dy_dev)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pkg.scan_bwd(*args, dy_dev, out=out)
    for r in range(3):
        t = make_random_inputs(*shape, seed=82 + r)
        dy, _ = make_dy(t, "f32", 90 + r)
        with torch.cuda.stream(s):
            _copy_inputs(args, t)
            dy_dev.copy_(torch.from_numpy(np.asarray(dy, dtype=np.float32)))
            for k in NAMES:
                out[k].fill_(float("nan"))
        g.replay()
        s.synchronize()
        got = {k: as_f64(v) for k, v in out.items()}
        check_grads(got, oracle.bwd(*(t[k] for k in KEYS), dy), "f32", shape[3] * shape[4], f"bwd replay {r}")
    pkg.sync_check(s)


@pytest.mark.parametrize("waves", [None, "1"])
def test_epoch_wrap_across_a_shape_change(waves, monkeypatch):
    """A launch leaves tagged carry words in the ring; 65535 launches later
    the tags repeat. Forced here with the test hook: a large map runs with
    stored epoch 0 (tag 1), a smaller map wraps the epoch (the ring is
    cleared), and the large map runs again with tag 1 on new inputs. Without
    the clear it would take the first run's words where the smaller map did
    not overwrite them."""
    if waves:
        monkeypatch.setenv("SSM2D_WAVES", waves)
    big, small = (1, 32, 16, 64, 512), (1, 16, 16, 16, 96)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        t1 = make_random_inputs(*big, seed=100)
        pkg.scan_fwd(*to_dev(t1, "f32"))  # creates the stream's workspace at the big size
        pkg.set_epoch_for_test(0, s)
        y1 = pkg.scan_fwd(*to_dev(t1, "f32"))
        s.synchronize()
        check(as_f64(y1), ref_of(t1), "f32", "big map, tag epoch 1")
        pkg.set_epoch_for_test(65533, s)
        ts = make_random_inputs(*small, seed=101)
        for k in range(2):  # stored 65533 -> 65534 -> 0 (wrap)
            ys = pkg.scan_fwd(*to_dev(ts, "f32"))
            s.synchronize()
            check(as_f64(ys), ref_of(ts), "f32", f"small map {k}")
        t2 = make_random_inputs(*big, seed=102)
        y2 = pkg.scan_fwd(*to_dev(t2, "f32"))
        s.synchronize()
        check(as_f64(y2), ref_of(t2), "f32", "big map again, tag epoch 1 after the wrap")
    pkg.sync_check(s)


def test_timeout_surfaces_on_the_next_call(monkeypatch):
    """A tiny bound on the kernels' own carry waits (the condition is forced
    from the host; every kernel still exits): a wait that gave up leaves NaN
    in the outputs from that point on, and the next call on the stream
    reports SSM2D_ERR_DEVICE_TIMEOUT without running; the call after that is
    exact again."""
    monkeypatch.setenv("SSM2D_WAVES", "1")
    shape = (1, 16, 16, 64, 128)
    t = make_random_inputs(*shape, seed=110)
    args = to_dev(t, "f32")
    pkg.set_spin_limit(1)
    try:
        y = pkg.scan_fwd(*args)
        torch.cuda.synchronize()
    finally:
        pkg.set_spin_limit(0)
    has_nan = bool(torch.isnan(y).any().item())
    try:
        y2 = pkg.scan_fwd(*args)
        reported = False
    except pkg.Ssm2dError as e:
        assert e.status == pkg.ERR_DEVICE_TIMEOUT
        reported = True
    _say(f"  forced wait bound: NaN outputs={has_nan}, reported on the next call={reported}")
    assert has_nan == reported
    if not reported:
        torch.cuda.synchronize()
        check(as_f64(y2), ref_of(t), "f32", "no timeout happened")
    pkg.sync_check()
    check(as_f64(pkg.scan_fwd(*args)), ref_of(t), "f32", "after the reported timeout")
    pkg.sync_check()


def test_release_workspaces_and_reuse():
    """Workspaces of a stream are freed and built again by the next call."""
    shape = (1, 16, 16, 33, 80)
    t = make_random_inputs(*shape, seed=120)
    dy, dy_dev = make_dy(t, "f32", 121)
    args = to_dev(t, "f32")
    for r in range(2):
        y = pkg.scan_fwd(*args)
        g = pkg.scan_bwd(*args, dy_dev)
        yb = pkg.scan_fwd_mamba(*args, delta_softplus=True)
        pkg.sync_check()
        check(as_f64(y), ref_of(t), "f32", f"forward, round {r}")
        check_grads({k: as_f64(v) for k, v in g.items()}, oracle.bwd(*(t[k] for k in KEYS), dy), "f32",
                    shape[3] * shape[4], f"backward, round {r}")
        check(as_f64(yb), oracle.fwd_mamba(*(t[k] for k in KEYS), delta_softplus=True), "f32", f"options, round {r}")
        pkg.release_workspaces()


# (SSM2D_RING, SSM2D_OVERFLOW, streams): the bounded ring with overflow rows
# (default), a slot a row, the bounded ring alone (tickets in blocks of 8
# chains: at most 120 waiting workgroups a launch, so two launches)
RING_MODES = [(None, None, 3), ("0", None, 3), ("32", "0", 2)]


@pytest.mark.parametrize("mode", RING_MODES, ids=str)
def test_concurrent_streams(mode, monkeypatch):
    """Streams each launch the giga-pixel map (384 x 512, 128 channels, 16
    states: chains across workgroups, a grid that alone fills the GPU)
    several times without waiting, so the launches compete for the compute
    units. Every launch drains: no wait gives up, and each output equals (bit
    for bit) the same call run alone; sampled maps match the oracle."""
    ring, ovf, nstreams = mode
    if ring:
        monkeypatch.setenv("SSM2D_RING", ring)
    if ovf:
        monkeypatch.setenv("SSM2D_OVERFLOW", ovf)
    shape = (1, 128, 16, 384, 512)
    assert pkg.fwd_kernels(*shape) == (1, 0, 0)
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    ts = [make_random_inputs(*shape, seed=130 + i) for i in range(nstreams)]
    args, alone = [], []
    for s, t in zip(streams, ts):
        with torch.cuda.stream(s):
            a = to_dev(t, "f32")
            args.append(a)
            alone.append(pkg.scan_fwd(*a))
        s.synchronize()
        pkg.sync_check(s)
    maps = [0, 63, 127]
    check(as_f64(alone[0]).reshape(-1, 384, 512)[maps], ref_of(ts[0], maps=maps), "f32", "giga-pixel map alone")
    outs = [[torch.empty_like(alone[i]) for _ in range(4)] for i in range(nstreams)]
    for r in range(4):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                pkg.scan_fwd(*args[i], y=outs[i][r])
    for i, s in enumerate(streams):
        s.synchronize()
        pkg.sync_check(s)
        for r in range(4):
            assert torch.equal(outs[i][r], alone[i]), f"stream {i} launch {r}"
    _say(f"  {4 * nstreams} overlapping launches on {nstreams} streams {mode}: all equal to the lone runs")


@pytest.mark.parametrize("shape", [(1, 128, 16, 384, 512), (2, 40, 16, 96, 512), (1, 16, 16, 80, 96)], ids=str)
@pytest.mark.parametrize("fast", ["1", "0"])
def test_overflow_rows(shape, fast, monkeypatch):
    """Every producer moves to the overflow rows after its first 8 rows
    (SSM2D_OVERFLOW=2; one-strip workgroups on the small map), through the
    two-rows-per-step forward and the general kernel: exact against the
    oracle on sampled maps, and bit for bit equal to the bounded ring's run."""
    monkeypatch.setenv("SSM2D_FAST", fast)
    if shape[4] < 512:
        monkeypatch.setenv("SSM2D_WAVES", "1")
    t = make_random_inputs(*shape, seed=150 + shape[3])
    args = to_dev(t, "f32")
    y0 = pkg.scan_fwd(*args)
    pkg.sync_check()
    monkeypatch.setenv("SSM2D_OVERFLOW", "2")
    _say(f"overflow rows {shape} fast={fast}")
    y = pkg.scan_fwd(*args)
    pkg.sync_check()
    assert torch.equal(y, y0)
    nmaps = shape[0] * shape[1]
    maps = sorted({0, nmaps // 2, nmaps - 1})
    check(as_f64(y).reshape(nmaps, shape[3], shape[4])[maps], ref_of(t, maps=maps), "f32", f"overflow {shape}")


@pytest.mark.parametrize("tblk", ["1", "3", "8", "64"])
def test_ticket_blocks(tblk, monkeypatch):
    """The bounded ring without overflow rows, tickets dealt in blocks of 1,
    3, 8 chains, and all chains at once (10 chains: a partial last block), through the
    two-rows-per-step forward and the general kernel; exact against the
    oracle on every map."""
    monkeypatch.setenv("SSM2D_OVERFLOW", "0")
    monkeypatch.setenv("SSM2D_TICKET_BLOCK", tblk)
    shape = (2, 40, 16, 96, 512)
    t = make_random_inputs(*shape, seed=140 + int(tblk))
    args = to_dev(t, "f32")
    ref = ref_of(t)
    for fast in ("1", "0"):
        monkeypatch.setenv("SSM2D_FAST", fast)
        _say(f"ticket blocks of {tblk} chains, SSM2D_FAST={fast}")
        y = pkg.scan_fwd(*args)
        pkg.sync_check()
        check(as_f64(y), ref, "f32", f"tblk={tblk} fast={fast}")


@pytest.mark.parametrize("tblk", ["1", "8"])
def test_ticket_blocks_wide_chains(tblk, monkeypatch):
    """The giga-pixel map in 8-column strips across workgroups (4 strips and
    two couriers a workgroup) with the bounded ring alone, tickets dealt in
    blocks of 1 and 8 chains: bit for bit equal to the default plan's run,
    sampled maps exact against the oracle."""
    shape = (1, 128, 16, 384, 512)
    t = make_random_inputs(*shape, seed=150)
    args = to_dev(t, "f32")
    y0 = pkg.scan_fwd(*args)
    pkg.sync_check()
    monkeypatch.setenv("SSM2D_OVERFLOW", "0")
    monkeypatch.setenv("SSM2D_TICKET_BLOCK", tblk)
    assert pkg.fwd_kernels(*shape) == (1, 0, 0)
    _say(f"wide chains, ticket blocks of {tblk}")
    y = pkg.scan_fwd(*args)
    pkg.sync_check()
    assert torch.equal(y, y0)
    maps = [0, 77, 127]
    check(as_f64(y).reshape(128, 384, 512)[maps], ref_of(t, maps=maps), "f32", f"wide chains tblk={tblk}")
