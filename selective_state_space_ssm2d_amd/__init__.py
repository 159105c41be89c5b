"""MI355X (gfx950) 2D selective scan — Python binding of libssm2d.so.

This module only marshals arguments: it checks tensors, passes their device
pointers and the current HIP stream to the C ABI declared in
``include/ssm2d.h``, and turns status codes into exceptions. Every step of the
scan runs in the library's HIP kernels. PyTorch supplies device memory and
streams only. There is no fallback: if the library is missing the call fails.

    y = scan_fwd(x, delta, A, B, C, D)
    y = scan_fwd_ex(x, delta, A, B, C, D, flip_h=..., flip_w=..., vertical_first=...,
                    accumulate=..., four_way=...)
    y = scan_fwd_mamba(x, delta, A, B, C, D, z=..., delta_bias=..., delta_softplus=...)
    g = scan_bwd(x, delta, A, B, C, D, dy)   # dict: dx, ddelta, dA, dB, dC, dD

x, delta: [batch, d_inner, H, W]; B, C: [batch, d_state, H, W]; all four
float32 or all four bfloat16. A: [d_inner, d_state] float32; D: [d_inner]
float32 (``scan_fwd_ex``: or None, no skip term). y has the dtype of x. All
tensors on the current CUDA (HIP) device, contiguous. ``scan_fwd_ex`` selects
the scan direction and order, and multi-direction sums (SSM2D_* flags).
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "LIB_PATH", "HEADER_PATH", "load_library", "scan_fwd", "scan_fwd_ex", "scan_fwd_mamba", "scan_bwd",
    "scan_bwd_mamba",
    "status_string",
    "sync_check", "set_spin_limit", "release_workspaces", "set_epoch_for_test", "fwd_kernels", "exported_names",
    "Ssm2dError",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssm2d.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "ssm2d.h")

(OK, ERR_NULLPTR, ERR_BAD_DIM, ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_HIP, ERR_NOMEM, ERR_DEVICE_TIMEOUT,
 ERR_BAD_FLAGS, ERR_TOO_LARGE) = range(10)
FLIP_H, FLIP_W, VERTICAL_FIRST, ACCUMULATE, FOUR_WAY, DELTA_SOFTPLUS = 1, 2, 4, 8, 16, 32

_lib = None


class Ssm2dError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def load_library(path: str = LIB_PATH):
    """Load libssm2d.so and declare the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    for name in ("ssm2d_scan_fwd", "ssm2d_scan_fwd_bf16", "ssm2d_scan_fwd_noalloc"):
        f = getattr(lib, name)
        f.argtypes = [vp] * 7 + [i64] * 5 + [vp]
        f.restype = ctypes.c_int
    for name in ("ssm2d_scan_fwd_mamba", "ssm2d_scan_fwd_mamba_bf16"):
        f = getattr(lib, name)
        f.argtypes = [vp] * 13 + [i64] * 5 + [ctypes.c_uint32, vp]
        f.restype = ctypes.c_int
    for name in ("ssm2d_scan_bwd_mamba", "ssm2d_scan_bwd_mamba_bf16"):
        f = getattr(lib, name)
        f.argtypes = [vp] * 23 + [i64] * 5 + [ctypes.c_uint32, vp]
        f.restype = ctypes.c_int
    for name in ("ssm2d_scan_bwd", "ssm2d_scan_bwd_bf16"):
        f = getattr(lib, name)
        f.argtypes = [vp] * 13 + [i64] * 5 + [vp]
        f.restype = ctypes.c_int
    for name in ("ssm2d_scan_bwd_ex", "ssm2d_scan_bwd_ex_bf16"):
        f = getattr(lib, name)
        f.argtypes = [vp] * 13 + [i64] * 5 + [ctypes.c_uint32, vp]
        f.restype = ctypes.c_int
    for name in ("ssm2d_scan_fwd_ex", "ssm2d_scan_fwd_ex_bf16"):
        f = getattr(lib, name)
        f.argtypes = [vp] * 7 + [i64] * 5 + [ctypes.c_uint32, vp]
        f.restype = ctypes.c_int
    lib.ssm2d_status_string.argtypes = [ctypes.c_int]
    lib.ssm2d_status_string.restype = ctypes.c_char_p
    lib.ssm2d_sync_check.argtypes = [vp]
    lib.ssm2d_sync_check.restype = ctypes.c_int
    lib.ssm2d_set_spin_limit.argtypes = [i64]
    lib.ssm2d_set_spin_limit.restype = ctypes.c_int
    lib.ssm2d_release_workspaces.argtypes = [vp]
    lib.ssm2d_release_workspaces.restype = ctypes.c_int
    lib.ssm2d_test_set_epoch.argtypes = [vp, ctypes.c_uint32]
    lib.ssm2d_test_set_epoch.restype = ctypes.c_int
    lib.ssm2d_fwd_kernels.argtypes = [ctypes.c_int] + [i64] * 5 + [ctypes.c_uint32, vp, vp, vp]
    lib.ssm2d_fwd_kernels.restype = ctypes.c_int
    lib.ssm2d_version.argtypes = []
    lib.ssm2d_version.restype = ctypes.c_int
    lib.ssm2d_last_hip_error.argtypes = []
    lib.ssm2d_last_hip_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def exported_names(header: str = HEADER_PATH):
    """Function names the header declares (for the symbol-export check)."""
    with open(header) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(ssm2d_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    try:
        return load_library().ssm2d_status_string(int(status)).decode()
    except RuntimeError:
        return f"status {status}"


def _stream_handle(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def sync_check(stream=None) -> None:
    """Wait for the stream; raise if a kernel reported a device-side timeout."""
    s = load_library().ssm2d_sync_check(_stream_handle(stream))
    if s != OK:
        raise Ssm2dError(s, "ssm2d_sync_check")


def set_spin_limit(polls: int) -> None:
    load_library().ssm2d_set_spin_limit(int(polls))


def release_workspaces(stream=None) -> None:
    """Wait for the stream and free the library's workspaces for it (current
    device); raise if a timeout was still unreported."""
    s = load_library().ssm2d_release_workspaces(_stream_handle(stream))
    if s != OK:
        raise Ssm2dError(s, "ssm2d_release_workspaces")


def set_epoch_for_test(epoch: int, stream=None) -> None:
    """Test hook: set the stored carry-tag epoch of the stream's workspace."""
    s = load_library().ssm2d_test_set_epoch(_stream_handle(stream), int(epoch))
    if s != OK:
        raise Ssm2dError(s, "ssm2d_test_set_epoch")


def fwd_kernels(batch, d_inner, d_state, H, W, bf16=False, flip_h=False, flip_w=False, vertical_first=False,
                accumulate=False, four_way=False, delta_softplus=False):
    """(launches of the two-rows-per-step forward, launches of the general
    kernel, launches of the whole-row kernel for narrow maps) that a forward
    call of these sizes and options makes (no gate, delta bias or carried
    states). Host-side planning only: no GPU needed."""
    flags = ((FLIP_H if flip_h else 0) | (FLIP_W if flip_w else 0) | (VERTICAL_FIRST if vertical_first else 0)
             | (ACCUMULATE if accumulate else 0) | (FOUR_WAY if four_way else 0)
             | (DELTA_SOFTPLUS if delta_softplus else 0))
    fast, general, narrow = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    s = load_library().ssm2d_fwd_kernels(int(bool(bf16)), batch, d_inner, d_state, H, W, flags,
                                         ctypes.byref(fast), ctypes.byref(general), ctypes.byref(narrow))
    if s != OK:
        raise Ssm2dError(s, "ssm2d_fwd_kernels")
    return fast.value, general.value, narrow.value


def _check(x, delta, A, B, C, D, y, need_d):
    import torch

    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x and B must be 4-D")
    batch, d_inner, H, W = x.shape
    d_state = B.shape[1]
    if delta.shape != x.shape:
        raise ValueError("delta must have the shape of x")
    if B.shape != (batch, d_state, H, W) or C.shape != B.shape:
        raise ValueError("B and C must be [batch, d_state, H, W]")
    if D is None and need_d:
        raise ValueError("D is required")
    if A.shape != (d_inner, d_state) or (D is not None and D.shape != (d_inner,)):
        raise ValueError("A must be [d_inner, d_state] and D [d_inner]")
    dt = x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    for name, t in (("delta", delta), ("B", B), ("C", C)):
        if t.dtype != dt:
            raise TypeError(f"{name} must have the dtype of x")
    for name, t in (("A", A), ("D", D)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if y is None:
        y = torch.empty_like(x)
    elif y.shape != x.shape or y.dtype != dt:
        raise ValueError("y must match x in shape and dtype")
    dev = x.device
    for t in (x, delta, A, B, C, D, y):
        if t is None:
            continue
        if t.device != dev or dev.type != "cuda":
            raise ValueError("all tensors must be on the same GPU device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    return y, (batch, d_inner, d_state, H, W)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else None)


def _call(fn, lib, dev, args):
    import torch

    with torch.cuda.device(dev):
        s = fn(*args)
    if s == ERR_HIP:
        raise Ssm2dError(s, f"{fn.__name__} ({lib.ssm2d_last_hip_error().decode()})")
    if s != OK:
        raise Ssm2dError(s, fn.__name__)


def scan_fwd(x, delta, A, B, C, D, y=None, stream=None):
    """y = 2D selective scan forward (see module docstring)."""
    import torch

    lib = load_library()
    y, dims = _check(x, delta, A, B, C, D, y, need_d=True)
    fn = lib.ssm2d_scan_fwd if x.dtype == torch.float32 else lib.ssm2d_scan_fwd_bf16
    _call(fn, lib, x.device, [_ptr(t) for t in (x, delta, A, B, C, D, y)] + [*dims, _stream_handle(stream)])
    return y


def scan_fwd_ex(x, delta, A, B, C, D=None, y=None, *, flip_h=False, flip_w=False, vertical_first=False,
                accumulate=False, four_way=False, flags=None, stream=None):
    """2D selective scan forward in another direction / order (include/ssm2d.h,
    ssm2d_scan_fwd_ex). With ``accumulate`` the result is added to ``y``, which
    must then be given. ``flags`` (an int of SSM2D_* bits) overrides the
    keyword switches and is passed through unchecked."""
    import torch

    lib = load_library()
    if accumulate and y is None:
        raise ValueError("accumulate needs y")
    y, dims = _check(x, delta, A, B, C, D, y, need_d=False)
    if flags is None:
        flags = ((FLIP_H if flip_h else 0) | (FLIP_W if flip_w else 0) | (VERTICAL_FIRST if vertical_first else 0)
                 | (ACCUMULATE if accumulate else 0) | (FOUR_WAY if four_way else 0))
    fn = lib.ssm2d_scan_fwd_ex if x.dtype == torch.float32 else lib.ssm2d_scan_fwd_ex_bf16
    _call(fn, lib, x.device, [_ptr(t) for t in (x, delta, A, B, C, D, y)] + [*dims, int(flags), _stream_handle(stream)])
    return y


def scan_fwd_mamba(x, delta, A, B, C, D=None, z=None, delta_bias=None, y=None, *, delta_softplus=False,
                   h_init=None, h_last=None, return_last_state=False, hh_init=None, hh_last=None,
                   return_last_row_state=False, flip_h=False, flip_w=False, vertical_first=False, four_way=False,
                   accumulate=False, stream=None):
    """The 2D scan with Mamba's operator options (include/ssm2d.h,
    ssm2d_scan_fwd_mamba): step size delta + delta_bias[d], optionally through
    softplus, the output gated by SiLU(z), carried vertical states (h_init in,
    h_last out; float32 [batch, d_inner, d_state, W]) and carried row states
    (hh_init in, hh_last out; float32 [batch, d_inner, d_state, H]). Returns
    y, or a tuple (y, h_last if return_last_state, hh_last if
    return_last_row_state)."""
    import torch

    lib = load_library()
    if accumulate and y is None:
        raise ValueError("accumulate needs y")
    y, dims = _check(x, delta, A, B, C, D, y, need_d=False)
    if z is not None and (z.shape != x.shape or z.dtype != x.dtype or z.device != x.device or not z.is_contiguous()):
        raise ValueError("z must match x in shape, dtype and device, and be contiguous")
    if delta_bias is not None and (delta_bias.shape != (dims[1],) or delta_bias.dtype != torch.float32
                                   or delta_bias.device != x.device):
        raise ValueError("delta_bias must be float32 [d_inner] on x's device")
    cshape = (dims[0], dims[1], dims[2], dims[4])
    rshape = (dims[0], dims[1], dims[2], dims[3])
    if return_last_state and h_last is None:
        h_last = torch.empty(cshape, dtype=torch.float32, device=x.device)
    if return_last_row_state and hh_last is None:
        hh_last = torch.empty(rshape, dtype=torch.float32, device=x.device)
    for name, t, shp, what in (("h_init", h_init, cshape, "W"), ("h_last", h_last, cshape, "W"),
                               ("hh_init", hh_init, rshape, "H"), ("hh_last", hh_last, rshape, "H")):
        if t is not None and (t.shape != shp or t.dtype != torch.float32 or t.device != x.device
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 [batch, d_inner, d_state, {what}] on x's device")
    flags = ((FLIP_H if flip_h else 0) | (FLIP_W if flip_w else 0) | (VERTICAL_FIRST if vertical_first else 0)
             | (ACCUMULATE if accumulate else 0) | (FOUR_WAY if four_way else 0)
             | (DELTA_SOFTPLUS if delta_softplus else 0))
    fn = lib.ssm2d_scan_fwd_mamba if x.dtype == torch.float32 else lib.ssm2d_scan_fwd_mamba_bf16
    _call(fn, lib, x.device, [_ptr(t) for t in (x, delta, A, B, C, D, z, delta_bias, h_init, h_last, hh_init, hh_last,
                                                 y)]
          + [*dims, flags, _stream_handle(stream)])
    out = (y,) + ((h_last,) if return_last_state else ()) + ((hh_last,) if return_last_row_state else ())
    return out if len(out) > 1 else y


def scan_bwd(x, delta, A, B, C, D, dy, out=None, stream=None, *, flip_h=False, flip_w=False,
             vertical_first=False):
    """Gradients of the forward scan for upstream gradient dy (include/ssm2d.h,
    ssm2d_scan_bwd; with flip_h / flip_w / vertical_first, ssm2d_scan_bwd_ex
    for the scan in that direction and order). Returns a dict dx, ddelta, dA,
    dB, dC, dD; ``out`` may supply any of them (shapes and dtypes as the
    inputs they belong to)."""
    import torch

    lib = load_library()
    _check(x, delta, A, B, C, D, None, need_d=True)
    if dy.shape != x.shape or dy.dtype != x.dtype or dy.device != x.device or not dy.is_contiguous():
        raise ValueError("dy must match x in shape, dtype and device, and be contiguous")
    batch, d_inner, H, W = x.shape
    d_state = B.shape[1]
    like = {"dx": x, "ddelta": delta, "dA": A, "dB": B, "dC": C, "dD": D}
    g = {}
    for k, ref in like.items():
        t = (out or {}).get(k)
        if t is None:
            t = torch.empty_like(ref)
        elif t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
            raise ValueError(f"{k} must match its input in shape, dtype and device, and be contiguous")
        g[k] = t
    args = [_ptr(t) for t in (x, delta, A, B, C, D, dy)] + [_ptr(g[k]) for k in ("dx", "ddelta", "dA", "dB", "dC", "dD")]
    if flip_h or flip_w or vertical_first:
        fn = lib.ssm2d_scan_bwd_ex if x.dtype == torch.float32 else lib.ssm2d_scan_bwd_ex_bf16
        flags = (FLIP_H if flip_h else 0) | (FLIP_W if flip_w else 0) | (VERTICAL_FIRST if vertical_first else 0)
        _call(fn, lib, x.device, args + [batch, d_inner, d_state, H, W, flags, _stream_handle(stream)])
    else:
        fn = lib.ssm2d_scan_bwd if x.dtype == torch.float32 else lib.ssm2d_scan_bwd_bf16
        _call(fn, lib, x.device, args + [batch, d_inner, d_state, H, W, _stream_handle(stream)])
    return g


def scan_bwd_mamba(x, delta, A, B, C, D, dy, z=None, delta_bias=None, *, delta_softplus=False, h_init=None,
                   dh_last=None, hh_init=None, dhh_last=None, flip_h=False, flip_w=False, vertical_first=False,
                   stream=None):
    """Gradients of scan_fwd_mamba (include/ssm2d.h, ssm2d_scan_bwd_mamba):
    scan_bwd's dict with ddelta taken with respect to the raw delta, plus dz
    (when z is given), ddelta_bias (when delta_bias is given), dh_init
    (when h_init or dh_last is given: the forward's carried vertical state
    and dL/dh_last, float32 [batch, d_inner, d_state, W]) and dhh_init (when
    hh_init or dhh_last is given: the carried row state and dL/dhh_last,
    float32 [batch, d_inner, d_state, H])."""
    import torch

    lib = load_library()
    _check(x, delta, A, B, C, D, None, need_d=True)
    if dy.shape != x.shape or dy.dtype != x.dtype or dy.device != x.device or not dy.is_contiguous():
        raise ValueError("dy must match x in shape, dtype and device, and be contiguous")
    if z is not None and (z.shape != x.shape or z.dtype != x.dtype or z.device != x.device or not z.is_contiguous()):
        raise ValueError("z must match x in shape, dtype and device, and be contiguous")
    batch, d_inner, H, W = x.shape
    if delta_bias is not None and (delta_bias.shape != (d_inner,) or delta_bias.dtype != torch.float32
                                   or delta_bias.device != x.device):
        raise ValueError("delta_bias must be float32 [d_inner] on x's device")
    d_state = B.shape[1]
    g = {"dx": torch.empty_like(x), "ddelta": torch.empty_like(delta), "dA": torch.empty_like(A),
         "dB": torch.empty_like(B), "dC": torch.empty_like(C), "dD": torch.empty_like(D)}
    if z is not None:
        g["dz"] = torch.empty_like(z)
    if delta_bias is not None:
        g["ddelta_bias"] = torch.empty_like(delta_bias)
    cshape, rshape = (batch, d_inner, d_state, W), (batch, d_inner, d_state, H)
    for name, t, shp, what in (("h_init", h_init, cshape, "W"), ("dh_last", dh_last, cshape, "W"),
                               ("hh_init", hh_init, rshape, "H"), ("dhh_last", dhh_last, rshape, "H")):
        if t is not None and (t.shape != shp or t.dtype != torch.float32 or t.device != x.device
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 [batch, d_inner, d_state, {what}] on x's device")
    if h_init is not None or dh_last is not None:
        g["dh_init"] = torch.empty(cshape, dtype=torch.float32, device=x.device)
    if hh_init is not None or dhh_last is not None:
        g["dhh_init"] = torch.empty(rshape, dtype=torch.float32, device=x.device)
    flags = ((DELTA_SOFTPLUS if delta_softplus else 0) | (FLIP_H if flip_h else 0) | (FLIP_W if flip_w else 0)
             | (VERTICAL_FIRST if vertical_first else 0))
    fn = lib.ssm2d_scan_bwd_mamba if x.dtype == torch.float32 else lib.ssm2d_scan_bwd_mamba_bf16
    args = [_ptr(t) for t in (x, delta, A, B, C, D, z, delta_bias, h_init, dh_last, hh_init, dhh_last, dy)] + \
        [_ptr(g.get(k)) for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh_init", "dhh_init")]
    _call(fn, lib, x.device, args + [batch, d_inner, d_state, H, W, flags, _stream_handle(stream)])
    return g
