"""fp64 CPU oracle for the 2DMamba 2D selective scan — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package. The product path (the HIP library and its Python
binding) never imports, loads or calls it, and shares no code with it.

The arithmetic lives in ``ssm2d_oracle.c`` (plain fp64 loops over the two
recurrences of the 2D selective scan, see that file's header for the equations
and the passages they follow). This module only marshals numpy arrays.

Functions
---------
build()                 compile ssm2d_oracle.c into libssm2d_oracle.so (gcc)
fwd(x, delta, A, B, C, D, maps=None, nthreads=0, flip_h=False, flip_w=False,
    vertical_first=False, four_way=False) -> y (float64)
states(abar, bx, flip_h=False, flip_w=False, vertical_first=False) -> h
                        the recurrences alone on given Abar, Bx (one map)
bwd(x, delta, A, B, C, D, dy, flip_h=False, flip_w=False, vertical_first=False)
                        -> dict of dx, ddelta, dA, dB, dC, dD (float64)
fwd_mamba(x, delta, A, B, C, D, z=None, delta_bias=None, delta_softplus=False, ...)
                        the scan with Mamba's step-size bias / softplus and SiLU(z) gating
bwd_mamba(x, delta, A, B, C, D, dy, z=None, delta_bias=None, delta_softplus=False)
                        its gradients (bwd's dict plus dz, ddelta_bias)
max_threads()           OpenMP thread count the oracle uses by default
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm2d_oracle.c")
LIB_PATH = os.path.join(_HERE, "libssm2d_oracle.so")

_lib = None


def build(out_path: str = LIB_PATH, src_path: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-std=c99", *extra_flags, src_path, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def load(path: str = LIB_PATH):
    """Load a compiled oracle library (default: the in-tree one)."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_ssm2d_fwd_maps_f64.argtypes = [dp] * 7 + [i64] * 5 + [
        ctypes.POINTER(i64), i64, ctypes.c_int]
    lib.oracle_ssm2d_fwd_maps_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_states_f64.argtypes = [dp, dp, dp, i64, i64]
    lib.oracle_ssm2d_states_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_fwd_ex_f64.argtypes = [dp] * 7 + [i64] * 5 + [
        ctypes.POINTER(i64), i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_ssm2d_fwd_ex_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_states_ex_f64.argtypes = [dp, dp, dp, i64, i64, ctypes.c_int]
    lib.oracle_ssm2d_states_ex_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_fwd_carry_f64.argtypes = [dp] * 9 + [i64] * 5 + [ctypes.c_int, ctypes.c_int]
    lib.oracle_ssm2d_fwd_carry_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_fwd_tile_f64.argtypes = [dp] * 11 + [i64] * 5 + [ctypes.c_int, ctypes.c_int]
    lib.oracle_ssm2d_fwd_tile_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_bwd_f64.argtypes = [dp] * 13 + [i64] * 5 + [ctypes.c_int]
    lib.oracle_ssm2d_bwd_carry_f64.argtypes = [dp] * 16 + [i64] * 5 + [ctypes.c_int]
    lib.oracle_ssm2d_bwd_carry_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_bwd_tile_f64.argtypes = [dp] * 19 + [i64] * 5 + [ctypes.c_int]
    lib.oracle_ssm2d_bwd_tile_f64.restype = ctypes.c_int
    lib.oracle_ssm2d_bwd_f64.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"oracle library {LIB_PATH} is not built; run __graft_entry__.build()")
        _lib = load(LIB_PATH)
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _flags(flip_h, flip_w, vertical_first):
    return (1 if flip_h else 0) | (2 if flip_w else 0) | (4 if vertical_first else 0)


def fwd(x, delta, A, B, C, D, maps=None, nthreads=0, lib=None, flip_h=False, flip_w=False,
        vertical_first=False, four_way=False, h_init=None, return_last=False, hh_init=None,
        return_last_col=False):
    """y = 2D selective scan forward in fp64.

    x, delta: [batch][d_inner][H][W]; A: [d_inner][d_state]; B, C:
    [batch][d_state][H][W]; D: [d_inner]. With ``maps`` (flat indices
    b*d_inner+d), returns y for those maps only, shape [len(maps)][H][W];
    otherwise the full [batch][d_inner][H][W]. flip_h / flip_w scan rows
    bottom to top / columns right to left; vertical_first runs the column
    recurrence before the row recurrence. four_way sums the scans from the
    four corners (the four-quadrant propagation of the juejin.cn page, part 七
    section 4) with the D x term counted once; D may be None (no skip term).
    h_init ([batch][d_inner][d_state][W], may be None) is the carried vertical
    state before the first row in scan order; return_last also returns the
    state after the last row (y, h_last): scanning a map in bands of rows
    with these carries gives the scan of the whole map. hh_init
    ([batch][d_inner][d_state][H], may be None) is the carried horizontal
    state (the row recurrence's carry) before the first column in scan
    order, by row; return_last_col also returns the state after the last
    column: bands of columns, and tiles with both carries, compose likewise.
    With both, the result is (y, h_last, hh_last).
    """
    if D is None:
        D = np.zeros(np.shape(A)[0])
    if four_way:
        assert not (flip_h or flip_w)
        zero = np.zeros_like(_f64(D))
        y = fwd(x, delta, A, B, C, D, maps, nthreads, lib, vertical_first=vertical_first)
        for fh, fw in ((True, False), (False, True), (True, True)):
            y = y + fwd(x, delta, A, B, C, zero, maps, nthreads, lib, flip_h=fh, flip_w=fw,
                        vertical_first=vertical_first)
        return y
    flags = _flags(flip_h, flip_w, vertical_first)
    lib = lib or _get()
    if h_init is not None or return_last or hh_init is not None or return_last_col:
        assert maps is None and not four_way
        x, delta, A, B, C, D = map(_f64, (x, delta, A, B, C, D))
        batch, d_inner, H, W = x.shape
        d_state = A.shape[1]
        y = np.empty((batch, d_inner, H, W), dtype=np.float64)
        hl = np.empty((batch, d_inner, d_state, W), dtype=np.float64)
        gl = np.empty((batch, d_inner, d_state, H), dtype=np.float64)
        h0 = None if h_init is None else _f64(h_init)
        g0 = None if hh_init is None else _f64(hh_init)
        assert h0 is None or h0.shape == hl.shape
        assert g0 is None or g0.shape == gl.shape
        null = ctypes.POINTER(ctypes.c_double)()
        s = lib.oracle_ssm2d_fwd_tile_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y),
                                          null if h0 is None else _ptr(h0), _ptr(hl),
                                          null if g0 is None else _ptr(g0), _ptr(gl), batch, d_inner, d_state,
                                          H, W, int(nthreads), flags)
        if s != 0:
            raise RuntimeError(f"oracle failed with status {s}")
        out = (y,) + ((hl,) if return_last else ()) + ((gl,) if return_last_col else ())
        return out if len(out) > 1 else y
    x, delta, A, B, C, D = map(_f64, (x, delta, A, B, C, D))
    batch, d_inner, H, W = x.shape
    d_state = A.shape[1]
    assert delta.shape == x.shape
    assert A.shape == (d_inner, d_state) and D.shape == (d_inner,)
    assert B.shape == (batch, d_state, H, W) and C.shape == B.shape
    if maps is None:
        y = np.empty((batch, d_inner, H, W), dtype=np.float64)
        mp, nm = None, batch * d_inner
    else:
        m = np.ascontiguousarray(maps, dtype=np.int64)
        y = np.empty((m.size, H, W), dtype=np.float64)
        mp, nm = m.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), m.size
    if flags == 0:
        s = lib.oracle_ssm2d_fwd_maps_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                          _ptr(D), _ptr(y), batch, d_inner, d_state, H, W,
                                          mp, nm, int(nthreads))
    else:
        s = lib.oracle_ssm2d_fwd_ex_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                        _ptr(D), _ptr(y), batch, d_inner, d_state, H, W,
                                        mp, nm, int(nthreads), flags)
    if s != 0:
        raise RuntimeError(f"oracle failed with status {s}")
    return y


def states(abar, bx, lib=None, flip_h=False, flip_w=False, vertical_first=False):
    """h for one state map from given Abar [H][W] and Bx [H][W] (fp64)."""
    lib = lib or _get()
    abar, bx = _f64(abar), _f64(bx)
    H, W = abar.shape
    h = np.empty((H, W), dtype=np.float64)
    flags = _flags(flip_h, flip_w, vertical_first)
    if flags == 0:
        s = lib.oracle_ssm2d_states_f64(_ptr(abar), _ptr(bx), _ptr(h), H, W)
    else:
        s = lib.oracle_ssm2d_states_ex_f64(_ptr(abar), _ptr(bx), _ptr(h), H, W, flags)
    if s != 0:
        raise RuntimeError(f"oracle failed with status {s}")
    return h


def softplus(v):
    """log(1 + e^v) in fp64, without overflow for large v."""
    v = np.asarray(v, dtype=np.float64)
    return np.where(v > 0, v + np.log1p(np.exp(-np.abs(v))), np.log1p(np.exp(v)))


def silu(z):
    """z * sigmoid(z) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def fwd_mamba(x, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
              maps=None, lib=None, **dirs):
    """The Mamba selective-scan operator's options around the 2D scan: the
    step size is delta + delta_bias[d] (bias per channel), passed through
    softplus when asked, and the output is gated by SiLU(z), z shaped like x
    (Mamba's selective_scan_fn options; the codewithpapers.app record lists
    that function as the official code's entry point). Everything in fp64.
    ``dirs``: flip_h, flip_w, vertical_first, four_way as for fwd."""
    dt = np.asarray(delta, dtype=np.float64)
    if delta_bias is not None:
        dt = dt + np.asarray(delta_bias, dtype=np.float64)[None, :, None, None]
    if delta_softplus:
        dt = softplus(dt)
    y = fwd(x, dt, A, B, C, D, maps=maps, lib=lib, **dirs)
    if z is not None:
        g = silu(z)
        if maps is not None:
            b_, d_, H, W = np.shape(x)
            g = g.reshape(b_ * d_, H, W)[np.asarray(maps)]
        y = y * g
    return y


def bwd_mamba(x, delta, A, B, C, D, dy, z=None, delta_bias=None, delta_softplus=False, lib=None, h_init=None,
              dh_last=None, hh_init=None, dhh_last=None, **dirs):
    """Gradients of fwd_mamba (step-size bias and softplus, SiLU(z) gate) for
    upstream dy, by the chain rule around the scan's backward: the gate gives
    dz = dy * y_scan * SiLU'(z) and hands dy * SiLU(z) to the scan; the step
    size hands d delta' back through softplus (its derivative is the logistic
    sigmoid) and sums it over cells for the bias. Everything in fp64.
    Returns the dict of bwd plus dz and ddelta_bias where they apply.
    h_init / dh_last, hh_init / dhh_last and the direction keywords (flip_h,
    flip_w, vertical_first) pass through to fwd and bwd (dh_init, dhh_init
    then in the dict)."""
    raw = np.asarray(delta, dtype=np.float64)
    pre = raw if delta_bias is None else raw + np.asarray(delta_bias, dtype=np.float64)[None, :, None, None]
    dt = softplus(pre) if delta_softplus else pre
    dyf = np.asarray(dy, dtype=np.float64)
    out = {}
    if z is not None:
        zf = np.asarray(z, dtype=np.float64)
        sig = 1.0 / (1.0 + np.exp(-zf))
        y_scan = fwd(x, dt, A, B, C, D, lib=lib, h_init=h_init, hh_init=hh_init, **dirs)
        out["dz"] = dyf * y_scan * sig * (1.0 + zf * (1.0 - sig))
        dyf = dyf * zf * sig
    g = bwd(x, dt, A, B, C, D, dyf, lib=lib, h_init=h_init, dh_last=dh_last, hh_init=hh_init, dhh_last=dhh_last,
            **dirs)
    dd = g["ddelta"]
    if delta_softplus:
        dd = dd / (1.0 + np.exp(-pre))
    g["ddelta"] = dd
    if delta_bias is not None:
        out["ddelta_bias"] = dd.sum(axis=(0, 2, 3))
    g.update(out)
    return g


def bwd(x, delta, A, B, C, D, dy, nthreads=0, lib=None, flip_h=False, flip_w=False, vertical_first=False,
        h_init=None, dh_last=None, hh_init=None, dhh_last=None):
    """Gradients of the forward pass (fp64) for upstream gradient dy (shape of
    y): returns dict dx, ddelta, dA, dB, dC, dD, each shaped like its input.
    flip_h / flip_w: of the scan in that direction, which is the upper-left
    scan of the mirrored map (a permutation of the cells), so its gradients
    are the mirrored map's, mirrored back. vertical_first: of the scan in the
    other order, which is the horizontal-first scan of the transposed map
    (cell (i, j) becomes (j, i); a flip of the rows becomes a flip of the
    columns and the other way round), so its gradients are the transposed
    map's, transposed back. Both identities are permutations of the cells;
    the finite-difference pins check the results independently.

    h_init / dh_last ([batch][d_inner][d_state][W], may be None): the
    backward of the forward with a carried vertical state h_init, for the
    loss sum(dy * y) + sum(dh_last * h_last); the result then also holds
    dh_init, shaped like h_init. hh_init / dhh_last ([batch][d_inner]
    [d_state][H]): the same for the carried row state (dhh_init). In the
    vertical-first order the two kinds trade places on the transposed map."""
    carry = h_init is not None or dh_last is not None
    rcarry = hh_init is not None or dhh_last is not None
    if vertical_first:
        tr = lambda a: np.ascontiguousarray(np.swapaxes(np.asarray(a, dtype=np.float64), 2, 3))
        g = bwd(tr(x), tr(delta), A, tr(B), tr(C), D, tr(dy), nthreads, lib, flip_h=flip_w, flip_w=flip_h,
                h_init=hh_init, dh_last=dhh_last, hh_init=h_init, dhh_last=dh_last)
        for k in ("dx", "ddelta", "dB", "dC"):
            g[k] = tr(g[k])
        g["dh_init"], g["dhh_init"] = g.pop("dhh_init", None), g.pop("dh_init", None)
        return {k: v for k, v in g.items() if v is not None}
        tr = lambda a: np.ascontiguousarray(np.swapaxes(np.asarray(a, dtype=np.float64), 2, 3))
        g = bwd(tr(x), tr(delta), A, tr(B), tr(C), D, tr(dy), nthreads, lib, flip_h=flip_w, flip_w=flip_h)
        for k in ("dx", "ddelta", "dB", "dC"):
            g[k] = tr(g[k])
        return g
    if flip_h or flip_w:
        ax = tuple(a for a, f in ((2, flip_h), (3, flip_w)) if f)
        fl = lambda a: np.ascontiguousarray(np.flip(np.asarray(a, dtype=np.float64), ax))

        def flc(a):  # carried states are per column: mirrored with the columns only
            if a is None or not flip_w:
                return a
            return np.ascontiguousarray(np.flip(np.asarray(a, dtype=np.float64), 3))

        def flr(a):  # carried row states are per row: mirrored with the rows only
            if a is None or not flip_h:
                return a
            return np.ascontiguousarray(np.flip(np.asarray(a, dtype=np.float64), 3))

        g = bwd(fl(x), fl(delta), A, fl(B), fl(C), D, fl(dy), nthreads, lib, h_init=flc(h_init),
                dh_last=flc(dh_last), hh_init=flr(hh_init), dhh_last=flr(dhh_last))
        for k in ("dx", "ddelta", "dB", "dC"):
            g[k] = fl(g[k])
        if "dh_init" in g:
            g["dh_init"] = flc(g["dh_init"])
        if "dhh_init" in g:
            g["dhh_init"] = flr(g["dhh_init"])
        return g
    lib = lib or _get()
    x, delta, A, B, C, D, dy = map(_f64, (x, delta, A, B, C, D, dy))
    batch, d_inner, H, W = x.shape
    d_state = A.shape[1]
    assert delta.shape == x.shape and dy.shape == x.shape
    assert A.shape == (d_inner, d_state) and D.shape == (d_inner,)
    assert B.shape == (batch, d_state, H, W) and C.shape == B.shape
    out = {"dx": np.empty_like(x), "ddelta": np.empty_like(x), "dA": np.empty_like(A),
           "dB": np.empty_like(B), "dC": np.empty_like(C), "dD": np.empty_like(D)}
    if carry or rcarry:
        cshape, rshape = (batch, d_inner, d_state, W), (batch, d_inner, d_state, H)
        h0 = None if h_init is None else _f64(h_init)
        gl = None if dh_last is None else _f64(dh_last)
        g0 = None if hh_init is None else _f64(hh_init)
        ggl = None if dhh_last is None else _f64(dhh_last)
        assert (h0 is None or h0.shape == cshape) and (gl is None or gl.shape == cshape)
        assert (g0 is None or g0.shape == rshape) and (ggl is None or ggl.shape == rshape)
        if carry:
            out["dh_init"] = np.empty(cshape, dtype=np.float64)
        if rcarry:
            out["dhh_init"] = np.empty(rshape, dtype=np.float64)
        null = ctypes.POINTER(ctypes.c_double)()
        p = lambda a: null if a is None else _ptr(a)
        s = lib.oracle_ssm2d_bwd_tile_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dy),
                                          p(h0), p(gl), p(g0), p(ggl),
                                          *(_ptr(out[k]) for k in ("dx", "ddelta", "dA", "dB", "dC", "dD")),
                                          p(out.get("dh_init")), p(out.get("dhh_init")), batch, d_inner, d_state,
                                          H, W, int(nthreads))
        if s != 0:
            raise RuntimeError(f"oracle failed with status {s}")
        return out
    s = lib.oracle_ssm2d_bwd_f64(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(dy),
                                 *(_ptr(out[k]) for k in ("dx", "ddelta", "dA", "dB", "dC", "dD")),
                                 batch, d_inner, d_state, H, W, int(nthreads))
    if s != 0:
        raise RuntimeError(f"oracle failed with status {s}")
    return out


def max_threads(lib=None) -> int:
    return int((lib or _get()).oracle_max_threads())
