"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/ssm2d.h declares, and validates arguments before any
HIP call (so these paths return their documented status codes here)."""
import ctypes
import os

import pytest

import selective_state_space_ssm2d_amd as pkg


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkg.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return pkg.load_library()


def test_exports_every_declared_symbol(lib):
    names = pkg.exported_names()
    assert "ssm2d_scan_fwd" in names and "ssm2d_scan_fwd_bf16" in names
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(10):
        text = lib.ssm2d_status_string(s)
        assert text and text != b"unknown status", s
    assert lib.ssm2d_status_string(99) == b"unknown status"
    assert lib.ssm2d_version() >= 300


FAKE = 0x10000  # never dereferenced: validation fails or returns first


def _call(lib, dims, ptrs=None, bf16=False):
    ptrs = ptrs if ptrs is not None else [FAKE] * 7
    fn = lib.ssm2d_scan_fwd_bf16 if bf16 else lib.ssm2d_scan_fwd
    return fn(*(ctypes.c_void_p(p) for p in ptrs), *dims, None)


@pytest.mark.parametrize("bf16", [False, True])
def test_negative_dims(lib, bf16):
    for k in range(5):
        dims = [1, 2, 3, 4, 5]
        dims[k] = -1
        assert _call(lib, dims, bf16=bf16) == pkg.ERR_BAD_DIM


@pytest.mark.parametrize("bf16", [False, True])
def test_zero_sizes_are_noops(lib, bf16):
    # nothing is launched, so even null pointers are fine
    for dims in ([0, 2, 3, 4, 5], [1, 0, 3, 4, 5], [1, 2, 3, 0, 5], [1, 2, 3, 4, 0]):
        assert _call(lib, dims, ptrs=[0] * 7, bf16=bf16) == pkg.OK


def test_unsupported_sizes(lib):
    assert _call(lib, [1, 2, 65, 4, 5]) == pkg.ERR_UNSUPPORTED
    assert _call(lib, [1, 2, 4, 65536, 5]) == pkg.ERR_UNSUPPORTED
    assert _call(lib, [1 << 16, 1 << 16, 4, 2, 1]) == pkg.ERR_UNSUPPORTED


def test_null_pointers(lib):
    for k in range(7):
        ptrs = [FAKE] * 7
        ptrs[k] = 0
        assert _call(lib, [1, 2, 3, 4, 5], ptrs) == pkg.ERR_NULLPTR, k
    # with d_state == 0, A, B and C are not read
    ptrs = [FAKE, FAKE, 0, 0, 0, FAKE, FAKE]
    assert _call(lib, [1, 2, 0, 4, 5], ptrs) != pkg.ERR_NULLPTR


def test_misaligned(lib):
    for k in range(7):
        ptrs = [FAKE] * 7
        ptrs[k] = FAKE + 4
        assert _call(lib, [1, 2, 3, 4, 5], ptrs) == pkg.ERR_MISALIGNED, k


def _call_ex(lib, dims, flags, ptrs=None, bf16=False):
    ptrs = ptrs if ptrs is not None else [FAKE] * 7
    fn = lib.ssm2d_scan_fwd_ex_bf16 if bf16 else lib.ssm2d_scan_fwd_ex
    return fn(*(ctypes.c_void_p(p) for p in ptrs), *dims, flags, None)


@pytest.mark.parametrize("bf16", [False, True])
def test_ex_flag_validation(lib, bf16):
    # unknown bits, and a four-way sum with a flip, are refused before anything else
    for flags in (64, 1 << 31, pkg.FOUR_WAY | pkg.FLIP_H, pkg.FOUR_WAY | pkg.FLIP_W):
        assert _call_ex(lib, [1, 2, 3, 4, 5], flags, bf16=bf16) == pkg.ERR_BAD_FLAGS, flags
        assert _call_ex(lib, [-1, 2, 3, 4, 5], flags, bf16=bf16) == pkg.ERR_BAD_FLAGS, flags
    # valid flags reach the usual checks
    for flags in range(64):
        if flags & pkg.FOUR_WAY and flags & (pkg.FLIP_H | pkg.FLIP_W):
            continue
        assert _call_ex(lib, [1, -2, 3, 4, 5], flags, bf16=bf16) == pkg.ERR_BAD_DIM, flags
        assert _call_ex(lib, [1, 2, 3, 0, 5], flags, ptrs=[0] * 7, bf16=bf16) == pkg.OK, flags
        assert _call_ex(lib, [1, 2, 65, 4, 5], flags, bf16=bf16) == pkg.ERR_UNSUPPORTED, flags


def _call_mamba(lib, dims, flags, ptrs=None, bf16=False):
    ptrs = ptrs if ptrs is not None else [FAKE] * 9
    ptrs = ptrs[:8] + [0, 0, 0, 0] + ptrs[8:]  # no carried states
    fn = lib.ssm2d_scan_fwd_mamba_bf16 if bf16 else lib.ssm2d_scan_fwd_mamba
    return fn(*(ctypes.c_void_p(p) for p in ptrs), *dims, flags, None)


@pytest.mark.parametrize("bf16", [False, True])
def test_mamba_entry_validation(lib, bf16):
    # a gate cannot be combined with accumulation; unknown bits are refused
    assert _call_mamba(lib, [1, 2, 3, 4, 5], pkg.ACCUMULATE, bf16=bf16) == pkg.ERR_BAD_FLAGS
    assert _call_mamba(lib, [1, 2, 3, 4, 5], 64, bf16=bf16) == pkg.ERR_BAD_FLAGS
    ptrs = [FAKE] * 9
    ptrs[6] = 0  # no gate: accumulation is fine
    assert _call_mamba(lib, [1, 2, 3, 4, 5], pkg.ACCUMULATE, ptrs, bf16=bf16) not in (pkg.ERR_BAD_FLAGS, pkg.ERR_NULLPTR)
    # z, delta_bias and D are optional; the others are not
    ptrs = [FAKE] * 9
    ptrs[5] = ptrs[6] = ptrs[7] = 0
    assert _call_mamba(lib, [1, 2, 3, 4, 5], pkg.DELTA_SOFTPLUS, ptrs, bf16=bf16) not in (pkg.ERR_NULLPTR,
                                                                                         pkg.ERR_MISALIGNED)
    for k in (0, 1, 2, 3, 4, 8):
        ptrs = [FAKE] * 9
        ptrs[k] = 0
        assert _call_mamba(lib, [1, 2, 3, 4, 5], 0, ptrs, bf16=bf16) == pkg.ERR_NULLPTR, k
    for k in range(9):
        ptrs = [FAKE] * 9
        ptrs[k] = FAKE + 4
        assert _call_mamba(lib, [1, 2, 3, 4, 5], 0, ptrs, bf16=bf16) == pkg.ERR_MISALIGNED, k
    # carried states: optional, aligned, not with the four-corner sum
    fn = lib.ssm2d_scan_fwd_mamba_bf16 if bf16 else lib.ssm2d_scan_fwd_mamba
    base = [FAKE] * 6 + [0, 0]
    call = lambda hi, hl, flags: fn(*(ctypes.c_void_p(p) for p in base + [hi, hl, 0, 0, FAKE]), 1, 2, 3, 4, 5, flags,
                                    None)
    assert call(FAKE, FAKE, pkg.FOUR_WAY) == pkg.ERR_BAD_FLAGS
    assert call(FAKE + 4, 0, 0) == pkg.ERR_MISALIGNED and call(0, FAKE + 4, 0) == pkg.ERR_MISALIGNED
    assert call(FAKE, FAKE, pkg.FLIP_H | pkg.VERTICAL_FIRST) not in (pkg.ERR_BAD_FLAGS, pkg.ERR_MISALIGNED,
                                                                     pkg.ERR_NULLPTR)
    # carried row states: optional, aligned, not with a gate, accumulation or the four-corner sum
    rcall = lambda gi, gl, z, flags: fn(*(ctypes.c_void_p(p) for p in [FAKE] * 6 + [z, 0, 0, 0, gi, gl, FAKE]),
                                        1, 2, 3, 4, 5, flags, None)
    for flags in (pkg.FOUR_WAY, pkg.ACCUMULATE):
        assert rcall(FAKE, 0, 0, flags) == pkg.ERR_BAD_FLAGS and rcall(0, FAKE, 0, flags) == pkg.ERR_BAD_FLAGS
    assert rcall(FAKE, FAKE, FAKE, 0) == pkg.ERR_BAD_FLAGS  # gated
    assert rcall(FAKE + 4, 0, 0, 0) == pkg.ERR_MISALIGNED and rcall(0, FAKE + 4, 0, 0) == pkg.ERR_MISALIGNED
    assert rcall(FAKE, FAKE, 0, pkg.FLIP_H | pkg.FLIP_W | pkg.VERTICAL_FIRST | pkg.DELTA_SOFTPLUS) not in (
        pkg.ERR_BAD_FLAGS, pkg.ERR_MISALIGNED, pkg.ERR_NULLPTR)


def test_ex_null_and_misaligned(lib):
    # D may be NULL in the flag-taking entry points (no skip term) ...
    ptrs = [FAKE] * 7
    ptrs[5] = 0
    assert _call_ex(lib, [1, 2, 3, 4, 5], 0, ptrs) not in (pkg.ERR_NULLPTR, pkg.ERR_MISALIGNED)
    # ... but not in the plain one
    assert _call(lib, [1, 2, 3, 4, 5], ptrs) == pkg.ERR_NULLPTR
    for k in (0, 1, 2, 3, 4, 6):
        ptrs = [FAKE] * 7
        ptrs[k] = 0
        assert _call_ex(lib, [1, 2, 3, 4, 5], pkg.FLIP_W, ptrs) == pkg.ERR_NULLPTR, k
    for k in range(7):
        ptrs = [FAKE] * 7
        ptrs[k] = FAKE + 8
        assert _call_ex(lib, [1, 2, 3, 4, 5], pkg.VERTICAL_FIRST, ptrs) == pkg.ERR_MISALIGNED, k


def _call_bwd(lib, dims, ptrs=None, bf16=False):
    ptrs = ptrs if ptrs is not None else [FAKE] * 13
    fn = lib.ssm2d_scan_bwd_bf16 if bf16 else lib.ssm2d_scan_bwd
    return fn(*(ctypes.c_void_p(p) for p in ptrs), *dims, None)


@pytest.mark.parametrize("bf16", [False, True])
def test_bwd_validation(lib, bf16):
    for k in range(5):
        dims = [1, 2, 3, 4, 5]
        dims[k] = -1
        assert _call_bwd(lib, dims, bf16=bf16) == pkg.ERR_BAD_DIM
    assert _call_bwd(lib, [1, 2, 65, 4, 5], bf16=bf16) == pkg.ERR_UNSUPPORTED   # d_state > 64
    assert _call_bwd(lib, [1, 2, 33, 4, 5], bf16=bf16) not in (pkg.ERR_UNSUPPORTED, pkg.ERR_BAD_DIM)  # in chunks
    assert _call_bwd(lib, [1, 2, 4, 65536, 5], bf16=bf16) == pkg.ERR_UNSUPPORTED
    assert _call_bwd(lib, [1, 0, 3, 4, 5], ptrs=[0] * 13, bf16=bf16) == pkg.OK  # d_inner = 0: nothing
    # with d_state = 0, A, B, C, dA, dB, dC may be NULL
    ptrs = [FAKE] * 13
    for k in (2, 3, 4, 9, 10, 11):
        ptrs[k] = 0
    assert _call_bwd(lib, [1, 2, 0, 4, 5], ptrs, bf16=bf16) not in (pkg.ERR_NULLPTR, pkg.ERR_MISALIGNED)
    for k in range(13):
        ptrs = [FAKE] * 13
        ptrs[k] = 0
        assert _call_bwd(lib, [1, 2, 3, 4, 5], ptrs, bf16=bf16) == pkg.ERR_NULLPTR, k
        ptrs[k] = FAKE + 4
        assert _call_bwd(lib, [1, 2, 3, 4, 5], ptrs, bf16=bf16) == pkg.ERR_MISALIGNED, k


@pytest.mark.parametrize("bf16", [False, True])
def test_bwd_ex_validation(lib, bf16):
    fn = lib.ssm2d_scan_bwd_ex_bf16 if bf16 else lib.ssm2d_scan_bwd_ex
    call = lambda dims, flags, ptrs=None: fn(*(ctypes.c_void_p(p) for p in (ptrs or [FAKE] * 13)), *dims, flags, None)
    for flags in (pkg.ACCUMULATE, pkg.FOUR_WAY, pkg.DELTA_SOFTPLUS, 128):
        assert call([1, 2, 3, 4, 5], flags) == pkg.ERR_BAD_FLAGS, flags
    for flags in (pkg.FLIP_H, pkg.FLIP_W, pkg.FLIP_H | pkg.FLIP_W, pkg.VERTICAL_FIRST,
                  pkg.VERTICAL_FIRST | pkg.FLIP_H | pkg.FLIP_W):
        assert call([1, -2, 3, 4, 5], flags) == pkg.ERR_BAD_DIM
        assert call([1, 0, 3, 4, 5], flags, [0] * 13) == pkg.OK


@pytest.mark.parametrize("bf16", [False, True])
def test_bwd_mamba_validation(lib, bf16):
    fn = lib.ssm2d_scan_bwd_mamba_bf16 if bf16 else lib.ssm2d_scan_bwd_mamba
    call = lambda ptrs, dims, flags: fn(*(ctypes.c_void_p(p) for p in ptrs), *dims, flags, None)
    # x delta A B C D z bias h_init dh_last hh_init dhh_last dy | dx ddelta dA dB dC dD dz dbias dh_init dhh_init
    full = [FAKE] * 23
    for flags in (pkg.ACCUMULATE, pkg.FOUR_WAY, 128):
        assert call(full, [1, 2, 3, 4, 5], flags) == pkg.ERR_BAD_FLAGS, flags
    assert call(full, [1, -2, 3, 4, 5], pkg.FLIP_H | pkg.FLIP_W | pkg.VERTICAL_FIRST) == pkg.ERR_BAD_DIM
    assert call([0] * 23, [1, 0, 3, 4, 5], 0) == pkg.OK                   # d_inner = 0: nothing to do
    # carried states: aligned
    for k in (8, 9, 10, 11, 21, 22):
        odd = list(full)
        odd[k] = FAKE + 4
        assert call(odd, [1, 2, 3, 4, 5], 0) == pkg.ERR_MISALIGNED, k
    no_dz = list(full)
    no_dz[19] = 0
    assert call(no_dz, [1, 2, 3, 4, 5], 0) == pkg.ERR_NULLPTR             # z given, dz missing
    no_bias = list(full)
    no_bias[7] = 0
    assert call(no_bias, [1, 2, 3, 4, 5], 0) == pkg.ERR_NULLPTR           # d bias asked without a bias
    odd = list(full)
    odd[6] = FAKE + 4
    assert call(odd, [1, 2, 3, 4, 5], 0) == pkg.ERR_MISALIGNED


def test_python_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 3, 4)
    B = torch.zeros(1, 5, 3, 4)
    A, D = torch.zeros(2, 5), torch.zeros(2)
    with pytest.raises(ValueError):
        pkg.scan_fwd(x, x, A, B[:, :, :2], B, D)
    with pytest.raises(TypeError):
        pkg.scan_fwd(x.double(), x.double(), A, B.double(), B.double(), D)
    with pytest.raises(ValueError):  # CPU tensors are refused: no host fallback
        pkg.scan_fwd(x, x, A, B, B, D)
    with pytest.raises(ValueError):
        pkg.scan_fwd_ex(x, x, A, B, B, None, flip_w=True)
    with pytest.raises(ValueError):  # accumulating needs an output to add to
        pkg.scan_fwd_ex(x, x, A, B, B, D, accumulate=True)
    with pytest.raises(ValueError):  # the plain entry point needs D
        pkg.scan_fwd(x, x, A, B, B, None)


def test_fwd_kernels_query(lib, monkeypatch):
    """ssm2d_fwd_kernels: host-side planning only (no GPU), one count per scan
    launch: the two-rows-per-step kernel for the plain forward of rows of a
    multiple of 4 columns whose chains span workgroups (every such layout
    with SSM2D_FAST=2), the whole-row kernel for the plain forward of narrow
    maps (short, or a batch of at least 256 waves, every tensor under 2^31
    bytes; every narrow map with SSM2D_NARROW=2, none with 0), the general kernel for direction/order bits,
    ragged rows and SSM2D_FAST=0; argument errors as the forward's."""
    assert pkg.fwd_kernels(1, 128, 16, 384, 512) == (1, 0, 0)
    assert pkg.fwd_kernels(32, 192, 16, 56, 56, bf16=True) == (0, 1, 0)   # chains in one workgroup
    assert pkg.fwd_kernels(1, 128, 16, 384, 512, flip_h=True) == (1, 0, 0)
    assert pkg.fwd_kernels(1, 128, 16, 384, 512, flip_w=True) == (0, 1, 0)
    assert pkg.fwd_kernels(1, 128, 16, 384, 512, vertical_first=True) == (0, 1, 0)
    assert pkg.fwd_kernels(1, 128, 16, 384, 510) == (0, 1, 0)   # rows of 2 mod 4 columns
    assert pkg.fwd_kernels(64, 768, 16, 14, 14) == (0, 0, 1)     # 3072 waves of 16 channels
    assert pkg.fwd_kernels(64, 768, 16, 14, 14, flip_h=True) == (0, 0, 1)
    assert pkg.fwd_kernels(64, 768, 16, 14, 14, flip_w=True) == (0, 1, 0)
    assert pkg.fwd_kernels(64, 768, 16, 14, 14, four_way=True) == (0, 3, 1)
    assert pkg.fwd_kernels(64, 768, 17, 14, 14) == (0, 1, 0)     # more than 16 states
    assert pkg.fwd_kernels(64, 768, 16, 14, 17) == (0, 1, 0)     # more than 16 columns
    assert pkg.fwd_kernels(1, 16, 16, 4096, 16) == (0, 1, 0)     # one tall map: strips
    assert pkg.fwd_kernels(1, 16, 16, 128, 16) == (0, 0, 1)      # a short one: whole rows
    # the whole-row kernel addresses its tensors with 32-bit buffer offsets:
    # x of 4096 x 1024 x 14 x 14 is 3.3 GB in fp32 (strips), 1.6 GB in bf16
    assert pkg.fwd_kernels(4096, 1024, 16, 14, 14) == (0, 1, 0)
    assert pkg.fwd_kernels(4096, 1024, 16, 14, 14, bf16=True) == (0, 0, 1)
    fast, general, narrow = pkg.fwd_kernels(1, 128, 16, 384, 512, four_way=True)
    assert (fast, general, narrow) == (1, 3, 0)   # the first corner is the plain scan
    assert sum(pkg.fwd_kernels(32, 192, 16, 56, 56, bf16=True, four_way=True)) == 4
    assert pkg.fwd_kernels(0, 128, 16, 384, 512) == (0, 0, 0)
    monkeypatch.setenv("SSM2D_FAST", "0")
    assert pkg.fwd_kernels(1, 128, 16, 384, 512) == (0, 1, 0)
    monkeypatch.setenv("SSM2D_FAST", "2")
    assert pkg.fwd_kernels(32, 192, 16, 56, 56, bf16=True) == (1, 0, 0)
    assert pkg.fwd_kernels(1, 4, 4, 8, 8) == (0, 0, 1)
    monkeypatch.setenv("SSM2D_NARROW", "0")
    assert pkg.fwd_kernels(1, 4, 4, 8, 8) == (1, 0, 0)
    monkeypatch.delenv("SSM2D_FAST")
    assert pkg.fwd_kernels(1, 4, 4, 8, 8) == (0, 1, 0)
    monkeypatch.setenv("SSM2D_NARROW", "2")
    assert pkg.fwd_kernels(1, 16, 16, 4096, 16) == (0, 0, 1)
    monkeypatch.delenv("SSM2D_NARROW")
    with pytest.raises(pkg.Ssm2dError):
        pkg.fwd_kernels(1, 8, 16, 8, 8, flip_h=True, four_way=True)
    with pytest.raises(pkg.Ssm2dError):
        pkg.fwd_kernels(1, -8, 16, 8, 8)
    with pytest.raises(pkg.Ssm2dError):
        pkg.fwd_kernels(1, 8, 65, 8, 8)
    two, gen, nar = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert lib.ssm2d_fwd_kernels(0, 1, 8, 16, 8, 8, 1 << 10, ctypes.byref(two), ctypes.byref(gen),
                                 ctypes.byref(nar)) == pkg.ERR_BAD_FLAGS
    assert lib.ssm2d_fwd_kernels(0, 1, 8, 16, 8, 8, 0, None, ctypes.byref(gen), ctypes.byref(nar)) == pkg.ERR_NULLPTR
    assert lib.ssm2d_fwd_kernels(0, 1, 8, 16, 8, 8, 0, ctypes.byref(two), ctypes.byref(gen), None) == pkg.ERR_NULLPTR
