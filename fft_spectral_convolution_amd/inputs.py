"""Seeded synthetic inputs for the spectral convolution.

This module only draws random numbers; it holds none of the operator's
arithmetic.  The tests, the benchmark and the oracle checks all draw their
inputs here, so the HIP path and the oracle always see identical fp32 /
complex64 arrays.

Workloads (shapes follow the pages' workloads; no dataset is read):

* ``c1``  2D, B=2,   Cin=Cout=4,  32x32,     mx=my=8,  x ~ U[-1,1]
* ``c2``  2D, B=16,  Cin=Cout=32, 64x64,     mx=my=16, x = smooth random field
* ``c3``  2D, B=32,  Cin=Cout=64, 128x128,   mx=my=32, x ~ U[-1,1]
  (shaped like the 128x128 PDE step of the TurboFNO blog, section 5.1)
* ``c4``  1D, B=256, Cin=Cout=64, N=4096,    modes=64, x ~ N(0,1)
  (global token mixing along a sequence, FFT blog section 3.2)
* ``c5``  2D, B=2,   Cin=Cout=16, 2048x2048, mx=my=64, x ~ U[-1,1]
  (the 2048x2048 grid with a 64x64 low-mode block of the TurboFNO blog,
  sections 2.1-2.2)

Recipe: ``numpy.random.default_rng(seed)``; draw x first, then W.real, then
W.imag, each as one array in C order.  W = (N(0,1) + i N(0,1)) / (Cin*Cout).
The smooth field draws p, q (integers in [0,8)), a ~ U[0.5,1] and
phi ~ U[0,2 pi) as [B,C,8] arrays in that order, then the N(0, 0.01) noise.
"""

from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Config", "CONFIGS", "make_inputs", "make_weight", "make_x"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    kind: str          # "2d" or "1d"
    B: int
    Cin: int
    Cout: int
    H: int             # 1 for 1d
    W: int             # sequence length N for 1d
    mx: int            # 1 for 1d (one weight block)
    my: int            # modes for 1d
    dist: str          # "uniform", "normal" or "smooth"

    @property
    def x_shape(self):
        if self.kind == "1d":
            return (self.B, self.Cin, self.W)
        return (self.B, self.Cin, self.H, self.W)

    @property
    def out_shape(self):
        if self.kind == "1d":
            return (self.B, self.Cout, self.W)
        return (self.B, self.Cout, self.H, self.W)

    @property
    def w_shape(self):
        if self.kind == "1d":
            return (self.my, self.Cin, self.Cout)
        return (2, self.mx, self.my, self.Cin, self.Cout)

    @property
    def compulsory_bytes(self) -> int:
        """x + W + out, each touched once."""
        n = 1
        for s in self.x_shape:
            n *= s
        m = 1
        for s in self.out_shape:
            m *= s
        k = 1
        for s in self.w_shape:
            k *= s
        return 4 * n + 4 * m + 8 * k

    def describe(self) -> str:
        if self.kind == "1d":
            return (f"1D spectral conv B={self.B} Cin={self.Cin} Cout={self.Cout} "
                    f"N={self.W} modes={self.my}")
        return (f"2D spectral conv B={self.B} Cin={self.Cin} Cout={self.Cout} "
                f"{self.H}x{self.W} modes {self.mx}x{self.my}")


CONFIGS = {
    "c1": Config("c1", "2d", 2, 4, 4, 32, 32, 8, 8, "uniform"),
    "c2": Config("c2", "2d", 16, 32, 32, 64, 64, 16, 16, "smooth"),
    "c3": Config("c3", "2d", 32, 64, 64, 128, 128, 32, 32, "uniform"),
    "c4": Config("c4", "1d", 256, 64, 64, 1, 4096, 1, 64, "normal"),
    "c5": Config("c5", "2d", 2, 16, 16, 2048, 2048, 64, 64, "uniform"),
}


def make_x(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    """Draw the input field (float64 draws, returned as float32)."""
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(size=shape).astype(np.float32)
    if dist == "smooth":
        b, c, h, w = shape
        p = rng.integers(0, 8, size=(b, c, 8))
        q = rng.integers(0, 8, size=(b, c, 8))
        a = rng.uniform(0.5, 1.0, size=(b, c, 8))
        phi = rng.uniform(0.0, 2.0 * np.pi, size=(b, c, 8))
        noise = rng.normal(0.0, 0.01, size=shape)
        hh = np.arange(h, dtype=np.float64)[:, None]
        ww = np.arange(w, dtype=np.float64)[None, :]
        field = np.zeros(shape, dtype=np.float64)
        for j in range(8):
            ang = 2.0 * np.pi * (p[:, :, j, None, None] * hh / h + q[:, :, j, None, None] * ww / w)
            field += a[:, :, j, None, None] * np.sin(ang + phi[:, :, j, None, None])
        return (field + noise).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_weight(rng: np.random.Generator, shape, cin: int, cout: int) -> np.ndarray:
    """W = (N(0,1) + i N(0,1)) / (Cin*Cout) as complex64; real part drawn first."""
    re = rng.standard_normal(size=shape) / (cin * cout)
    im = rng.standard_normal(size=shape) / (cin * cout)
    return (re + 1j * im).astype(np.complex64)


def make_inputs(cfg, seed: int = 0):
    """(x float32, W complex64) for a Config or a config name, seeded."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng(seed)
    x = make_x(rng, cfg.x_shape, cfg.dist)
    w = make_weight(rng, cfg.w_shape, cfg.Cin, cfg.Cout)
    return x, w
