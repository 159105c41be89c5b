"""ssm2d_scan_fwd_noalloc: the forward in a static device array, through the C
ABI, against the allocating entry point ssm2d_scan_fwd (same kernels and
arithmetic; on the giga-pixel map the array holds a bounded carry ring where
the allocating call has a slot a row, which carries the same values: bitwise
equal) and the oracle, on two calls in a row, the second on a smaller map;
and a map whose workspace exceeds the array is refused before anything
runs."""
import ctypes

import numpy as np
import pytest

import selective_state_space_ssm2d_amd as pkg
from selective_state_space_ssm2d_amd.inputs import WORKLOADS, make_inputs, make_random_inputs
from test_gpu_parity import KEYS, _say, _setup, as_f64, check, ref_of, to_dev  # noqa: F401 (_setup: fixture)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _noalloc(args, y, dims):
    fn = pkg.load_library().ssm2d_scan_fwd_noalloc
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (*args, y)]
    stream = ctypes.c_void_p(int(torch.cuda.current_stream().cuda_stream))
    return fn(*ptrs, *dims, stream)


def _dims(t):
    b, d, H, W = t["x"].shape
    return [b, d, t["B"].shape[1], H, W]


def test_noalloc_matches_the_allocating_entry_point():
    wl = next(w for w in WORKLOADS if w.name == "gigapixel_wsi")
    cases = [("gigapixel_wsi", make_inputs(wl, seed=0)),
             ("smaller map, chains across workgroups", make_random_inputs(1, 16, 16, 40, 96, seed=130))]
    for name, t in cases:
        _say(f"noalloc: {name} {t['x'].shape}")
        args = to_dev(t, "f32")
        y_ref = pkg.scan_fwd(*args)
        y = torch.full_like(args[0], float("nan"))
        st = _noalloc(args, y, _dims(t))
        assert st == pkg.OK, pkg.status_string(st)
        pkg.sync_check()
        assert torch.equal(y, y_ref), name
        H, W = t["x"].shape[2:]
        nmaps = t["x"].shape[0] * t["x"].shape[1]
        maps = np.unique(np.array([0, nmaps // 2, nmaps - 1]))
        check(as_f64(y).reshape(nmaps, H, W)[maps], ref_of(t, maps=maps), "f32", f"noalloc {name} vs oracle")


def test_noalloc_refuses_a_map_beyond_the_scratch():
    """A zero page of more than the array's 1 MiB (H * W > 262128 cells)."""
    t = make_random_inputs(1, 8, 4, 600, 512, seed=131)
    args = to_dev(t, "f32")
    y = torch.full_like(args[0], 3.0)
    st = _noalloc(args, y, _dims(t))
    torch.cuda.synchronize()
    assert st == pkg.ERR_TOO_LARGE, pkg.status_string(st)
    assert bool((y == 3.0).all().item())
