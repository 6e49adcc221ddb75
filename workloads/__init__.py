"""Seeded synthetic inputs shaped like the video-DiT attention workloads on the pages.

This module is shared test and benchmark infrastructure. It holds none of the
method's arithmetic (no reordering, pooling, scoring, routing or attention): it
only draws q, k, v and rounds them to bf16.

Shapes follow the FVAttn review (xllm-io paper review of FVAttn, section
"五、实验结果 / 实验设置"): 720p video is 21 latent frames of 3,600 tokens. The
long-video shape is six times that horizon, after the LVSA note (wiki note on
LVSA, its summary of the 6x horizon experiments). Activations of the real models
are not available, so q and k carry a positional locality signal built from
random Fourier features (RFF) of the latent cell (t, y, x), plus i.i.d. noise:

    phi_h(x)[m] = sqrt(2) * cos(Omega_h[m] . x + b_h[m]),  m = 0..63
    Omega_h[m] ~ N(0, diag(1/l_t^2, 1/l_y^2, 1/l_x^2)),  b_h[m] ~ U[0, 2 pi)
    q[n, h, 0:64] = s_h * phi_h(x_n) + eps,  q[n, h, 64:d] = eps   (k alike, own eps)
    v ~ N(0, 1)

so that phi_h(x).phi_h(x') ~ 64 exp(-|Lambda (x - x')|^2 / 2): heads with a large
s_h attend locally (peaked block scores), heads with a small s_h are near-flat.
The length scales l = (2, 4, 4) cells are this generator's choice; the pages give
none.

Draw order (numpy Generator(PCG64(seed)), seed = config index): s_h; then per
head Omega_h and b_h; then q noise, k noise, v. Everything is drawn in float32
(float64 for the RFF phases) and rounded once to bf16 (round to nearest even);
that bf16 tensor is the single input to both the GPU path and the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

RFF_FEATURES = 64
LENGTH_SCALES = (2.0, 4.0, 4.0)  # cells along (t, y, x)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: grid, heads, block size and operating point."""

    index: int
    name: str
    B: int
    H: int
    d: int
    T: int
    Y: int
    X: int
    block: int
    p: float
    k_floor: int
    slack_frac: float = 0.0
    lpt: bool = False             # the configuration names the longest-first queue
    dtype: str = "bf16"          # "fp32" for the tiny case, else "bf16"
    s_mode: str = "loguniform"   # how the per-head signal scale s_h is drawn
    p_sweep: Sequence[float] = ()

    @property
    def N(self) -> int:
        return self.T * self.Y * self.X

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)

    @property
    def tiles(self) -> int:
        return self.B * self.H * self.nb


# The five workloads: a tiny fp32 case, Wan-1.3B-like 480p, Wan-14B-like 720p,
# a 720p head-skew stress case, and a 6x-horizon long video.
WORKLOADS = (
    Workload(0, "tiny-fp32", 1, 2, 64, 4, 8, 8, 16, 0.9, 2, dtype="fp32", s_mode="tiny"),
    Workload(1, "480p-12h", 1, 12, 128, 21, 30, 52, 64, 0.9, 4),
    Workload(2, "720p-40h", 1, 40, 128, 21, 45, 80, 64, 0.9, 4),
    Workload(3, "720p-40h-skew", 1, 40, 128, 21, 45, 80, 64, 0.95, 4,
             slack_frac=0.05, lpt=True, s_mode="skew"),
    Workload(4, "long6x-12h", 1, 12, 128, 126, 30, 52, 128, 0.9, 8,
             p_sweep=(0.8, 0.9, 0.95)),
)


def workload(index_or_name) -> Workload:
    for w in WORKLOADS:
        if w.index == index_or_name or w.name == index_or_name:
            return w
    raise KeyError(index_or_name)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _signal_scales(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.s_mode == "tiny":
        s = np.array([0.5, 3.0], dtype=np.float64)
        assert w.H == 2
        return s
    if w.s_mode == "skew":
        # heads 0..34 light (peaked, s = 5), heads 35..39 heavy (near-flat, s = 0.3)
        s = np.full(w.H, 5.0)
        s[w.H - 5:] = 0.3
        return s
    return np.exp(rng.uniform(math.log(0.5), math.log(4.0), size=w.H))


def cell_coords(T: int, Y: int, X: int) -> np.ndarray:
    """[N, 3] float64 cell coordinates (t, y, x), token n = (t*Y + y)*X + x."""
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)


def generate(w: Workload, seed: Optional[int] = None, want_fp32: bool = False):
    """Draw q, k, v of shape [B, N, H, d] in grid (row-major cell) order.

    Returns a dict with
      q16, k16, v16 : uint16 bf16 bits (the tensors both sides consume),
      q32, k32, v32 : the float32 draws before rounding (only if want_fp32),
      s             : float64 per-head signal scales.
    """
    seed = w.index if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    B, N, H, d = w.B, w.N, w.H, w.d
    s = _signal_scales(w, rng)
    omegas, phases = [], []
    inv_l = 1.0 / np.asarray(LENGTH_SCALES)
    for _ in range(H):
        omegas.append(rng.standard_normal((RFF_FEATURES, 3)) * inv_l)
        phases.append(rng.uniform(0.0, 2.0 * math.pi, size=RFF_FEATURES))
    pos = cell_coords(w.T, w.Y, w.X)

    nf = min(RFF_FEATURES, d)
    out = {"s": s}
    for name in ("q", "k"):
        x = rng.standard_normal((B, N, H, d), dtype=np.float32)
        for h in range(H):
            phi = (math.sqrt(2.0) * np.cos(pos @ omegas[h].T + phases[h])).astype(np.float32)
            x[:, :, h, :nf] += np.float32(s[h]) * phi[None, :, :nf]
        out[name + "16"] = bf16_bits(x)
        if want_fp32:
            out[name + "32"] = x
        del x
    v = rng.standard_normal((B, N, H, d), dtype=np.float32)
    out["v16"] = bf16_bits(v)
    if want_fp32:
        out["v32"] = v
    return out
