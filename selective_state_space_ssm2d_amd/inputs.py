"""Seeded synthetic inputs for the 2D selective scan.

This module is shared by the GPU path's tests/bench and by the fp64 oracle's
tests. It holds only the input recipe (random draws, casts, pad masks) and none
of the scan's arithmetic.

Tensor layout (row-major, W fastest):
    x, delta : [batch][d_inner][H][W]
    B, C     : [batch][d_state][H][W]   (selective, shared across d_inner)
    A        : [d_inner][d_state]       (fp32, negative)
    D        : [d_inner]                (fp32)

Recipe (the pages fix only the shapes of the workloads, not their values):
    draw order from numpy default_rng(seed): x, z, A_log, B, C, D
    x ~ N(0,1); delta = softplus(z), z ~ N(0,1); A = -exp(U[log 1, log 16]);
    B, C ~ N(0,1); D ~ N(0,1). Draws are fp64, rounded to fp32 (RNE).
    bf16 workloads additionally round x, delta, B, C to bf16 (RNE).
    Pad cells (non-tissue positions of a whole-slide grid) take one fixed
    vector drawn from default_rng(seed + 1): x <- p_x, delta <- softplus(p_z),
    B <- p_B, C <- p_C. The pad mask comes from default_rng(seed + 2).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "make_random_inputs",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "pad_mask",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    d_inner: int
    d_state: int
    H: int
    W: int
    dtype: str  # "f32" or "bf16" (bf16 = x, delta, B, C, y in bf16; A, D fp32)
    pad: Optional[str] = None  # None | "uniform" | "blob"
    pad_cells: int = 0

    @property
    def elements(self) -> int:
        return self.batch * self.d_inner * self.H * self.W


# The five workloads, in order: tiny; WSI multiple-instance map with 40 % pad
# cells; VMamba-T stage-1 shape in bf16; 14x14 padding-stress grid; giga-pixel
# WSI grid with 60 % blob-shaped pad cells.
WORKLOADS = [
    Workload("tiny", 1, 4, 4, 8, 8, "f32"),
    Workload("wsi_mil", 1, 128, 16, 64, 80, "f32", pad="uniform", pad_cells=2048),
    Workload("vmamba_t_s1", 32, 192, 16, 56, 56, "bf16"),
    Workload("grid14", 64, 768, 16, 14, 14, "f32"),
    Workload("gigapixel_wsi", 1, 128, 16, 384, 512, "f32", pad="blob", pad_cells=117965),
]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact fp32 value of bf16 bits."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, z)


def pad_mask(wl: Workload, seed: int = 0) -> Optional[np.ndarray]:
    """Boolean [H][W] mask of pad (non-tissue) cells, or None."""
    if wl.pad is None:
        return None
    n = wl.H * wl.W
    rng = np.random.default_rng(seed + 2)
    flat = np.zeros(n, dtype=bool)
    if wl.pad == "uniform":
        flat[rng.permutation(n)[: wl.pad_cells]] = True
    elif wl.pad == "blob":
        from scipy.ndimage import gaussian_filter

        noise = rng.standard_normal((wl.H, wl.W))
        field = gaussian_filter(noise, sigma=24.0, mode="wrap")
        order = np.argsort(field.ravel(), kind="stable")
        flat[order[: wl.pad_cells]] = True
    else:
        raise ValueError(wl.pad)
    return flat.reshape(wl.H, wl.W)


def _draw(rng, batch, d_inner, d_state, H, W):
    x = rng.standard_normal((batch, d_inner, H, W))
    z = rng.standard_normal((batch, d_inner, H, W))
    a_log = rng.uniform(np.log(1.0), np.log(16.0), size=(d_inner, d_state))
    Bm = rng.standard_normal((batch, d_state, H, W))
    Cm = rng.standard_normal((batch, d_state, H, W))
    Dv = rng.standard_normal((d_inner,))
    return x, z, a_log, Bm, Cm, Dv


def _finish(x, delta, A, Bm, Cm, Dv, dtype):
    out = {
        "A": np.ascontiguousarray(A, dtype=np.float32),
        "D": np.ascontiguousarray(Dv, dtype=np.float32),
    }
    for name, v in (("x", x), ("delta", delta), ("B", Bm), ("C", Cm)):
        f = np.ascontiguousarray(v, dtype=np.float32)
        if dtype == "bf16":
            bits = bf16_bits_from_f32(f)
            out[name + "_bits"] = bits
            f = f32_from_bf16_bits(bits)
        out[name] = f
    out["dtype"] = dtype
    return out


def make_inputs(wl: Workload, seed: int = 0) -> dict:
    """Inputs for one workload.

    Returns a dict with fp32 arrays x, delta, A, B, C, D holding the exact
    values the kernel sees (for bf16 workloads these are the bf16 values,
    widened), plus x_bits, delta_bits, B_bits, C_bits (uint16) for bf16
    workloads, and "mask" (bool [H][W] or None).
    """
    rng = np.random.default_rng(seed)
    x, z, a_log, Bm, Cm, Dv = _draw(rng, wl.batch, wl.d_inner, wl.d_state, wl.H, wl.W)
    delta = _softplus(z)
    del z
    A = -np.exp(a_log)
    mask = pad_mask(wl, seed)
    if mask is not None:
        prng = np.random.default_rng(seed + 1)
        p_x = prng.standard_normal(wl.d_inner)
        p_dt = _softplus(prng.standard_normal(wl.d_inner))
        p_B = prng.standard_normal(wl.d_state)
        p_C = prng.standard_normal(wl.d_state)
        ii, jj = np.nonzero(mask)
        x[:, :, ii, jj] = p_x[None, :, None]
        delta[:, :, ii, jj] = p_dt[None, :, None]
        Bm[:, :, ii, jj] = p_B[None, :, None]
        Cm[:, :, ii, jj] = p_C[None, :, None]
    out = _finish(x, delta, A, Bm, Cm, Dv, wl.dtype)
    out["mask"] = mask
    return out


def make_random_inputs(batch, d_inner, d_state, H, W, seed=0, dtype="f32",
                       a_range=(1.0, 16.0), delta_mode="softplus") -> dict:
    """Inputs of an arbitrary shape with the same value recipe.

    a_range: |A| ~ exp(U[log lo, log hi]); delta_mode: "softplus" (default),
    or "const" (one delta value per (b, d) map, drawn from the same
    distribution: the position-independent case).
    """
    rng = np.random.default_rng(seed)
    x, z, a_log, Bm, Cm, Dv = _draw(rng, batch, d_inner, d_state, H, W)
    lo, hi = a_range
    A = -np.exp(np.log(lo) + (a_log - np.log(1.0)) / np.log(16.0) * (np.log(hi) - np.log(lo)))
    if delta_mode == "const":
        z = np.broadcast_to(z[:, :, :1, :1], z.shape).copy()
    elif delta_mode != "softplus":
        raise ValueError(delta_mode)
    delta = _softplus(z)
    out = _finish(x, delta, A, Bm, Cm, Dv, dtype)
    out["mask"] = None
    return out
