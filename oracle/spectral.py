"""fp64 CPU oracle for the Fourier-neural-operator spectral convolution.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only
the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library (no
kernels, tables, constants or helpers) and never imports the package that
wraps the library.

Sources (the three web pages this method is described on):

* P1 -- "TurboFNO: FFT-GEMM-iFFT full-chain fused GPU operator" (gsyq.cn):
  section 1 (FFT -> frequency-domain GEMM -> iFFT chain), section 2.2 (only the
  low-frequency block of the spectrum is multiplied by the weights, the rest is
  zero; complex product (a+bi)(c+di) = (ac-bd) + (ad+bc)i), sections 3.1/4.4
  (orthonormal normalisation, scale 1/sqrt(M*N) on each transform).
* P2 -- "FFT for operator optimisation" (lpnh.cn): section 1.2 (convolution
  theorem), sections 2.1/2.2 (real-to-complex half spectrum of length N/2+1 on
  the last axis, complex-to-real inverse), section 6.4 (dump intermediate
  spectra from a Python reference and compare them point by point).

What is computed (all in float64 / complex128; fp32 / complex64 inputs are
upcast exactly):

1. forward, ortho:  X[b,i,kx,ky] = (HW)^-1/2 sum_h sum_w x[b,i,h,w]
                                    exp(-2 pi i (kx h / H + ky w / W))
2. truncate:  Xh[b,i,0,r,ky] = X[b,i,r,ky],  Xh[b,i,1,r,ky] = X[b,i,H-mx+r,ky]
              for r < mx, ky < my
3. mix:  Yh[b,o,s,r,ky] = sum_i Xh[b,i,s,r,ky] * W[s,r,ky,i,o]   (no conjugate)
4. zero-fill + complex-to-real inverse, ortho:
     out[b,o,h,w] = (HW)^-1/2 sum_kx sum_{ky<=W/2} c_ky
                      Re( Y[b,o,kx,ky] exp(+2 pi i (kx h / H + ky w / W)) )
   with c_0 = c_{W/2} = 1 and c_ky = 2 otherwise (the standard C2R rule: the
   imaginary parts of the DC and Nyquist columns do not contribute).
5. 1D: the same with H = 1, one weight block W[modes, Cin, Cout].
6. gradients of a real loss with dL/dout = g (the backward pass):
     dL/dx = the chain 1-4 applied to g with the conjugate-transposed weight
             W^H[s,r,ky,o,i] = conj W[s,r,ky,i,o];
     dL/dRe W + i dL/dIm W [s,r,ky,i,o] = c_ky sum_b conj(Xh[b,i,s,r,ky]) Gh[b,o,s,r,ky],
   Gh the truncated forward transform of g (derived below
   ``spectral_conv2d_backward_ref``; pinned by the adjoint identity and the
   exact change of the loss under weight perturbations).
7. fused layer tail (P2 sections 5.1-5.2: the C2R output is activated with
   GELU and added to a second, time-domain branch; section 6.2: fuse what
   follows the C2R into the same kernel):
     branch before the activation:  out = gelu(conv + bias[o] + branch)
     branch after the activation:   out = gelu(conv + bias[o]) + branch
   gelu(u) = u Phi(u) = u (1 + erf(u / sqrt 2)) / 2, the exact form (the page
   names GELU without choosing between it and its tanh approximation).
8. diagonal global filter / token mixer (P1 section 5.2: fft2 -> learnable
   mask -> ifft2 on a 512 x 512 image; P2 section 3.2: R2C along the
   sequence -> learnable complex mask -> C2R): one complex weight per kept
   mode and channel, no channel mixing,
     Yh[b,c,s,r,ky] = Xh[b,c,s,r,ky] * M[s,r,ky,c]   (1D: M[ky,c]),
   then step 4.  Keeping every mode (mx = H/2, my = W/2 + 1) gives the
   untruncated global filter.
9. zero-padded linear convolution (P2 sections 2.1 and 5.1-5.2: pad input
   and kernel, R2C, pointwise product, C2R, crop): the plain definition
     y[b,o,p,q] = sum_i sum_{dh<kh, dw<kw} x[b,i,p-dh,q-dw] k[o,i,dh,dw]
   (x zero outside its grid; y of size (H+kh-1) x (W+kw-1)), cropped to
   out = y[:, :, ch:ch+Ho, cw:cw+Wo].  The convolution theorem makes this
   the circular convolution on any grid of at least that size, which the
   GPU path computes with the spectral convolution at full modes.

Two independent ways of computing the transforms are provided:

* ``transform="dft"`` (default): the sums above written out as products with
  explicit DFT matrices whose phases come from the exact integer reduction
  (j*k) mod N.  This is the definition itself.
* ``transform="fft"``: full transforms by a textbook recursive radix-2
  decimation-in-time Cooley-Tukey FFT, then truncation; the inverse builds the
  Hermitian-extended row spectrum and transforms it.

``spectral_conv2d_loops`` is a pure-Python loop twin of the whole operator for
tiny sizes (brute force, no library transforms at all).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "dft_brute",
    "fft_radix2",
    "dft_matrix",
    "kept_kx",
    "c2r_weights",
    "forward_truncated_2d",
    "mix_2d",
    "inverse_from_truncated_2d",
    "spectral_conv2d_ref",
    "forward_truncated_1d",
    "mix_1d",
    "inverse_from_truncated_1d",
    "spectral_conv1d_ref",
    "spectral_conv2d_loops",
    "spectral_conv1d_loops",
    "spectral_conv2d_backward_ref",
    "spectral_conv1d_backward_ref",
    "gelu",
    "spectral_conv2d_gelu_ref",
    "spectral_conv1d_gelu_ref",
    "spectral_filter2d_ref",
    "spectral_filter1d_ref",
    "linear_conv2d_ref",
    "linear_conv1d_ref",
]


# --------------------------------------------------------------------------
# 1D transforms
# --------------------------------------------------------------------------

def _phase(m: np.ndarray, n: int, sign: int) -> np.ndarray:
    """exp(sign * 2 pi i * m / n) for integer m already reduced mod n."""
    ang = (2.0 * math.pi / n) * m.astype(np.float64)
    return np.cos(ang) + (1j * sign) * np.sin(ang)


def dft_matrix(n: int, rows: np.ndarray, cols: np.ndarray, sign: int) -> np.ndarray:
    """M[a, b] = exp(sign * 2 pi i * (rows[a] * cols[b] mod n) / n).

    The product of the two integer indices is reduced modulo n in integer
    arithmetic before it becomes an angle, so the phase is exact up to one
    rounding of cos/sin in float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    m = np.mod(np.outer(rows, cols), n)
    return _phase(m, n, sign)


def dft_brute(a: np.ndarray, axis: int = -1, sign: int = -1) -> np.ndarray:
    """Unnormalised O(N^2) DFT along ``axis``: A[k] = sum_n a[n] exp(sign 2 pi i n k / N)."""
    a = np.asarray(a, dtype=np.complex128)
    n = a.shape[axis]
    idx = np.arange(n)
    f = dft_matrix(n, idx, idx, sign)          # f[n, k]
    moved = np.moveaxis(a, axis, -1)
    out = moved @ f
    return np.moveaxis(out, -1, axis)


def fft_radix2(a: np.ndarray, axis: int = -1, sign: int = -1) -> np.ndarray:
    """Unnormalised recursive radix-2 decimation-in-time FFT along ``axis``.

    Textbook Cooley-Tukey: split into even and odd samples, transform each
    half, combine with the twiddles exp(sign 2 pi i k / N), k < N/2.
    N must be a power of two.
    """
    a = np.asarray(a, dtype=np.complex128)
    n = a.shape[axis]
    if n & (n - 1):
        raise ValueError(f"fft_radix2 needs a power-of-two length, got {n}")
    moved = np.moveaxis(a, axis, -1)

    def rec(v: np.ndarray) -> np.ndarray:
        m = v.shape[-1]
        if m == 1:
            return v.copy()
        even = rec(v[..., 0::2])
        odd = rec(v[..., 1::2])
        tw = _phase(np.arange(m // 2), m, sign) * odd
        return np.concatenate([even + tw, even - tw], axis=-1)

    return np.moveaxis(rec(moved), -1, axis)


def _real_times_complex(x: np.ndarray, m: np.ndarray) -> np.ndarray:
    """x @ m for real x[..., K] and complex m[K, J], as two real matrix products."""
    flat = np.ascontiguousarray(x, dtype=np.float64).reshape(-1, x.shape[-1])
    re = flat @ np.ascontiguousarray(m.real)
    im = flat @ np.ascontiguousarray(m.imag)
    return (re + 1j * im).reshape(x.shape[:-1] + (m.shape[1],))


def _real_part_of_product(a: np.ndarray, m: np.ndarray) -> np.ndarray:
    """Re(a @ m) for complex a[..., K] and complex m[K, J]."""
    flat = np.ascontiguousarray(a).reshape(-1, a.shape[-1])
    out = np.ascontiguousarray(flat.real) @ np.ascontiguousarray(m.real)
    out -= np.ascontiguousarray(flat.imag) @ np.ascontiguousarray(m.imag)
    return out.reshape(a.shape[:-1] + (m.shape[1],))


def _transform(a: np.ndarray, axis: int, sign: int, transform: str) -> np.ndarray:
    if transform == "dft":
        return dft_brute(a, axis, sign)
    if transform == "fft":
        return fft_radix2(a, axis, sign)
    raise ValueError(f"unknown transform {transform!r}")


# --------------------------------------------------------------------------
# Mode bookkeeping
# --------------------------------------------------------------------------

def kept_kx(h: int, mx: int) -> np.ndarray:
    """Frequencies along H kept by the truncation, in weight-block order.

    Block 0 holds kx = r and block 1 holds kx = H - mx + r, r < mx.
    """
    r = np.arange(mx)
    return np.concatenate([r, h - mx + r])


def c2r_weights(w: int, my: int) -> np.ndarray:
    """c_ky of the complex-to-real inverse: 1 at ky = 0 and ky = W/2, 2 elsewhere."""
    ky = np.arange(my)
    c = np.full(my, 2.0)
    c[ky == 0] = 1.0
    c[2 * ky == w] = 1.0
    return c


def _check_2d(h: int, w: int, mx: int, my: int) -> None:
    if mx < 1 or 2 * mx > h:
        raise ValueError(f"need 1 <= mx and 2*mx <= H (mx={mx}, H={h})")
    if my < 1 or my > w // 2 + 1:
        raise ValueError(f"need 1 <= my <= W/2+1 (my={my}, W={w})")


# --------------------------------------------------------------------------
# 2D operator, stage by stage
# --------------------------------------------------------------------------

def forward_truncated_2d(x: np.ndarray, mx: int, my: int, transform: str = "dft") -> np.ndarray:
    """Steps 1-2: ortho forward transform of real x[B,C,H,W], truncated to Xh[B,C,2,mx,my]."""
    x = np.asarray(x, dtype=np.float64)
    b, c, h, w = x.shape
    _check_2d(h, w, mx, my)
    scale = 1.0 / math.sqrt(h * w)
    kx = kept_kx(h, mx)
    if transform == "dft":
        fw = dft_matrix(w, np.arange(w), np.arange(my), -1)        # [W, my]
        fh = dft_matrix(h, kx, np.arange(h), -1)                   # [2mx, H]
        rows = _real_times_complex(x, fw)                          # [B,C,H,my]
        full = fh @ rows                                           # [B,C,2mx,my]
    else:
        rows = _transform(x.astype(np.complex128), 3, -1, transform)[..., :my]
        cols = _transform(rows, 2, -1, transform)                  # [B,C,H,my]
        full = cols[:, :, kx, :]
    return (full * scale).reshape(b, c, 2, mx, my)


def mix_2d(xh: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """Step 3: Yh[b,o,s,r,k] = sum_i Xh[b,i,s,r,k] W[s,r,k,i,o] (plain complex product)."""
    xh = np.asarray(xh, dtype=np.complex128)
    weight = np.asarray(weight, dtype=np.complex128)
    return np.einsum("bisrk,srkio->bosrk", xh, weight)


def inverse_from_truncated_2d(yh: np.ndarray, h: int, w: int, transform: str = "dft") -> np.ndarray:
    """Step 4: zero-fill Yh[B,C,2,mx,my] into the half spectrum and apply the ortho C2R inverse."""
    yh = np.asarray(yh, dtype=np.complex128)
    b, c, _, mx, my = yh.shape
    _check_2d(h, w, mx, my)
    scale = 1.0 / math.sqrt(h * w)
    kx = kept_kx(h, mx)
    yq = yh.reshape(b, c, 2 * mx, my)
    if transform == "dft":
        gh = dft_matrix(h, np.arange(h), kx, +1)                   # [H, 2mx]
        gw = dft_matrix(w, np.arange(my), np.arange(w), +1)        # [my, W]
        gw = gw * c2r_weights(w, my)[:, None]
        cols = gh @ yq                                             # [B,C,H,my]
        out = _real_part_of_product(cols, gw)                      # Re(cols @ gw)
        return out * scale
    # full half spectrum, zero outside the kept modes
    half = np.zeros((b, c, h, w // 2 + 1), dtype=np.complex128)
    half[:, :, kx, :my] = yq
    cols = _transform(half, 2, +1, transform)                      # inverse along H
    # Hermitian extension of every row, imaginary parts of DC / Nyquist dropped
    z = np.zeros((b, c, h, w), dtype=np.complex128)
    z[..., 1:w // 2] = cols[..., 1:w // 2]
    z[..., 0] = cols[..., 0].real
    z[..., w // 2] = cols[..., w // 2].real
    z[..., w // 2 + 1:] = np.conj(cols[..., 1:w // 2][..., ::-1])
    out = _transform(z, 3, +1, transform).real
    return out * scale


def spectral_conv2d_ref(x, weight, mx: int, my: int, transform: str = "dft",
                        return_stages: bool = False):
    """Whole 2D operator: x[B,Cin,H,W] real, weight[2,mx,my,Cin,Cout] complex -> out[B,Cout,H,W]."""
    x = np.asarray(x)
    weight = np.asarray(weight)
    _, cin, h, w = x.shape
    if weight.shape[:3] != (2, mx, my) or weight.shape[3] != cin:
        raise ValueError(f"weight shape {weight.shape} does not match (2,{mx},{my},{cin},Cout)")
    xh = forward_truncated_2d(x, mx, my, transform)
    yh = mix_2d(xh, weight)
    out = inverse_from_truncated_2d(yh, h, w, transform)
    if return_stages:
        return out, xh, yh
    return out


# --------------------------------------------------------------------------
# 1D operator (global token mixing along a sequence)
# --------------------------------------------------------------------------

def forward_truncated_1d(x: np.ndarray, modes: int, transform: str = "dft") -> np.ndarray:
    """Ortho forward transform of real x[B,C,N], bins ky < modes -> Xh[B,C,modes]."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if modes < 1 or modes > n // 2 + 1:
        raise ValueError(f"need 1 <= modes <= N/2+1 (modes={modes}, N={n})")
    scale = 1.0 / math.sqrt(n)
    if transform == "dft":
        full = _real_times_complex(x, dft_matrix(n, np.arange(n), np.arange(modes), -1))
    else:
        full = _transform(x.astype(np.complex128), -1, -1, transform)[..., :modes]
    return full * scale


def mix_1d(xh: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """Yh[b,o,k] = sum_i Xh[b,i,k] W[k,i,o]."""
    return np.einsum("bik,kio->bok", np.asarray(xh, np.complex128), np.asarray(weight, np.complex128))


def inverse_from_truncated_1d(yh: np.ndarray, n: int, transform: str = "dft") -> np.ndarray:
    """Zero-fill Yh[B,C,modes] and apply the ortho C2R inverse of length n."""
    yh = np.asarray(yh, dtype=np.complex128)
    modes = yh.shape[-1]
    scale = 1.0 / math.sqrt(n)
    if transform == "dft":
        g = dft_matrix(n, np.arange(modes), np.arange(n), +1) * c2r_weights(n, modes)[:, None]
        return _real_part_of_product(yh, g) * scale
    z = np.zeros(yh.shape[:-1] + (n,), dtype=np.complex128)
    half = np.zeros(yh.shape[:-1] + (n // 2 + 1,), dtype=np.complex128)
    half[..., :modes] = yh
    z[..., 1:n // 2] = half[..., 1:n // 2]
    z[..., 0] = half[..., 0].real
    z[..., n // 2] = half[..., n // 2].real
    z[..., n // 2 + 1:] = np.conj(half[..., 1:n // 2][..., ::-1])
    return _transform(z, -1, +1, transform).real * scale


def spectral_conv1d_ref(x, weight, modes: int, transform: str = "dft", return_stages: bool = False):
    """Whole 1D operator: x[B,Cin,N] real, weight[modes,Cin,Cout] complex -> out[B,Cout,N]."""
    x = np.asarray(x)
    weight = np.asarray(weight)
    if weight.shape[0] != modes or weight.shape[1] != x.shape[1]:
        raise ValueError(f"weight shape {weight.shape} does not match ({modes},{x.shape[1]},Cout)")
    xh = forward_truncated_1d(x, modes, transform)
    yh = mix_1d(xh, weight)
    out = inverse_from_truncated_1d(yh, x.shape[-1], transform)
    if return_stages:
        return out, xh, yh
    return out


# --------------------------------------------------------------------------
# Gradients (the backward pass of the same operator)
# --------------------------------------------------------------------------
#
# For a real loss L with g = dL/dout, write the operator as
#   out = sum_m c_m Re(Y_m phi_m),  Y_m = sum_i X_m,i W_m,i,o,
#   X_m = <x, phi_m> = sum_hw x conj(phi_m),  phi_m = (HW)^-1/2 exp(+2 pi i (kx h/H + ky w/W))
# (m runs over the kept modes, c_m the C2R weight of its ky).  With
# G_m = <g, phi_m> (the truncated forward transform of g):
#   dL/dx      = sum_m c_m Re(phi_m sum_o conj(W_m,i,o) G_m,o)
#              = the same forward -> mix -> inverse chain on g with the
#                conjugate-transposed weight W^H[m,o,i] = conj(W[m,i,o]);
#   dL/dRe W + i dL/dIm W = c_m sum_b conj(X_b,m,i) G_b,m,o.
# Both follow from dL = sum_m c_m Re(dY_m conj(G_m)) (the C2R weights enter
# the weight gradient only: in dL/dx the inverse applies them again).

def spectral_conv2d_backward_ref(x, weight, grad_out, mx: int, my: int, transform: str = "dft"):
    """Gradients of sum(grad_out * spectral_conv2d_ref(x, weight)).

    Returns (grad_x[B,Cin,H,W] float64, grad_w[2,mx,my,Cin,Cout] complex128),
    grad_w = dL/dRe(W) + i dL/dIm(W).
    """
    x = np.asarray(x)
    weight = np.asarray(weight, dtype=np.complex128)
    g = np.asarray(grad_out)
    _, cin, h, w = x.shape
    if weight.shape[:3] != (2, mx, my) or weight.shape[3] != cin or g.shape[1] != weight.shape[4]:
        raise ValueError(f"weight shape {weight.shape} does not match x {x.shape} / grad_out {g.shape}")
    xh = forward_truncated_2d(x, mx, my, transform)              # [B,Cin,2,mx,my]
    gh = forward_truncated_2d(g, mx, my, transform)              # [B,Cout,2,mx,my]
    zh = np.einsum("bosrk,srkio->bisrk", gh, np.conj(weight))     # G W^H
    grad_x = inverse_from_truncated_2d(zh, h, w, transform)
    c = c2r_weights(w, my)                                       # [my]
    grad_w = np.einsum("bisrk,bosrk->srkio", np.conj(xh), gh) * c[None, None, :, None, None]
    return grad_x, grad_w


def spectral_conv1d_backward_ref(x, weight, grad_out, modes: int, transform: str = "dft"):
    """Gradients of sum(grad_out * spectral_conv1d_ref(x, weight)).

    Returns (grad_x[B,Cin,N] float64, grad_w[modes,Cin,Cout] complex128).
    """
    x = np.asarray(x)
    weight = np.asarray(weight, dtype=np.complex128)
    g = np.asarray(grad_out)
    n = x.shape[-1]
    if weight.shape[0] != modes or weight.shape[1] != x.shape[1] or g.shape[1] != weight.shape[2]:
        raise ValueError(f"weight shape {weight.shape} does not match x {x.shape} / grad_out {g.shape}")
    xh = forward_truncated_1d(x, modes, transform)               # [B,Cin,modes]
    gh = forward_truncated_1d(g, modes, transform)               # [B,Cout,modes]
    zh = np.einsum("bok,kio->bik", gh, np.conj(weight))
    grad_x = inverse_from_truncated_1d(zh, n, transform)
    grad_w = np.einsum("bik,bok->kio", np.conj(xh), gh) * c2r_weights(n, modes)[:, None, None]
    return grad_x, grad_w


# --------------------------------------------------------------------------
# Fused layer tail: GELU and a second branch after the inverse transform
# --------------------------------------------------------------------------

def gelu(u):
    """u * Phi(u) with the standard normal CDF Phi(u) = (1 + erf(u / sqrt 2)) / 2."""
    from scipy.special import erf
    u = np.asarray(u, dtype=np.float64)
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def _layer_tail(y, bias, branch, branch_after: bool, channel_axis_shape):
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64).reshape(channel_axis_shape)
    if branch is not None and not branch_after:
        y = y + np.asarray(branch, dtype=np.float64)
    y = gelu(y)
    if branch is not None and branch_after:
        y = y + np.asarray(branch, dtype=np.float64)
    return y


def spectral_conv2d_gelu_ref(x, weight, mx: int, my: int, bias=None, branch=None, branch_after: bool = False,
                             transform: str = "dft"):
    """gelu(conv + bias[o] + branch), or gelu(conv + bias[o]) + branch when
    branch_after; conv = spectral_conv2d_ref(x, weight), bias [Cout] and
    branch [B,Cout,H,W] optional."""
    y = spectral_conv2d_ref(x, weight, mx, my, transform)
    return _layer_tail(y, bias, branch, branch_after, (1, -1, 1, 1))


def spectral_conv1d_gelu_ref(x, weight, modes: int, bias=None, branch=None, branch_after: bool = False,
                             transform: str = "dft"):
    """The 1D form of spectral_conv2d_gelu_ref (branch [B,Cout,N])."""
    y = spectral_conv1d_ref(x, weight, modes, transform)
    return _layer_tail(y, bias, branch, branch_after, (1, -1, 1))


# --------------------------------------------------------------------------
# Diagonal global filter: one complex weight per kept mode and channel
# --------------------------------------------------------------------------

def spectral_filter2d_ref(x, mask, mx: int, my: int, transform: str = "dft"):
    """out = C2R(truncate(R2C(x)) * mask), mask[2,mx,my,C] complex, x[B,C,H,W]."""
    x = np.asarray(x)
    mask = np.asarray(mask, dtype=np.complex128)
    _, c, h, w = x.shape
    if mask.shape != (2, mx, my, c):
        raise ValueError(f"mask shape {mask.shape} does not match (2, {mx}, {my}, {c})")
    xh = forward_truncated_2d(x, mx, my, transform)              # [B,C,2,mx,my]
    yh = xh * np.moveaxis(mask, -1, 0)[None]                     # [C,2,mx,my] per channel
    return inverse_from_truncated_2d(yh, h, w, transform)


def spectral_filter1d_ref(x, mask, modes: int, transform: str = "dft"):
    """The 1D form: mask[modes,C], x[B,C,N]."""
    x = np.asarray(x)
    mask = np.asarray(mask, dtype=np.complex128)
    _, c, n = x.shape
    if mask.shape != (modes, c):
        raise ValueError(f"mask shape {mask.shape} does not match ({modes}, {c})")
    xh = forward_truncated_1d(x, modes, transform)               # [B,C,modes]
    return inverse_from_truncated_1d(xh * mask.T[None], n, transform)


# --------------------------------------------------------------------------
# Linear (non-circular) convolution, by its definition
# --------------------------------------------------------------------------

def linear_conv2d_ref(x, k, crop_h: int = 0, crop_w: int = 0, out_h=None, out_w=None):
    """Full linear convolution of x[B,Cin,H,W] with k[Cout,Cin,kh,kw] (sum over
    Cin, kernel not flipped back: y[p] = sum x[p - d] k[d]), cropped to
    [crop_h : crop_h + out_h, crop_w : crop_w + out_w] (default: the rest)."""
    x = np.asarray(x, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    b, cin, h, w = x.shape
    cout, cin2, kh, kw = k.shape
    if cin2 != cin:
        raise ValueError(f"kernel {k.shape} does not match x {x.shape}")
    fh, fw = h + kh - 1, w + kw - 1
    y = np.zeros((b, cout, fh, fw))
    for dh in range(kh):
        for dw in range(kw):
            # every input pixel (p - dh, q - dw) lands at (p, q)
            y[:, :, dh:dh + h, dw:dw + w] += np.einsum("bihw,oi->bohw", x, k[:, :, dh, dw])
    out_h = fh - crop_h if out_h is None else out_h
    out_w = fw - crop_w if out_w is None else out_w
    if crop_h < 0 or crop_w < 0 or crop_h + out_h > fh or crop_w + out_w > fw:
        raise ValueError("crop window outside the full convolution")
    return y[:, :, crop_h:crop_h + out_h, crop_w:crop_w + out_w]


def linear_conv1d_ref(x, k, crop: int = 0, out_n=None):
    """The 1D form: x[B,Cin,N], k[Cout,Cin,K], full length N + K - 1."""
    x = np.asarray(x, dtype=np.float64)
    y = linear_conv2d_ref(x[:, :, None, :], np.asarray(k, dtype=np.float64)[:, :, None, :], 0, crop, 1, out_n)
    return y[:, :, 0, :]


# --------------------------------------------------------------------------
# Pure-Python loop twins (tiny sizes only)
# --------------------------------------------------------------------------

def spectral_conv2d_loops(x, weight, mx: int, my: int):
    """The whole 2D operator as explicit loops over every index (tiny inputs only).

    Each output sample is the sum over the kept modes of c_ky * Re(Y e^{+i phase})
    with Y the mixed spectrum; each spectrum entry is the double sum over the grid.
    """
    x = np.asarray(x, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.complex128)
    b_n, cin, h, w = x.shape
    cout = weight.shape[-1]
    _check_2d(h, w, mx, my)
    scale = 1.0 / math.sqrt(h * w)

    def e(sign, num, den):
        num %= den
        ang = 2.0 * math.pi * num / den
        return complex(math.cos(ang), sign * math.sin(ang))

    out = np.zeros((b_n, cout, h, w))
    for b in range(b_n):
        xh = {}
        for i in range(cin):
            for s in range(2):
                for r in range(mx):
                    kx = r if s == 0 else h - mx + r
                    for ky in range(my):
                        acc = 0j
                        for hh in range(h):
                            for ww in range(w):
                                acc += x[b, i, hh, ww] * e(-1, kx * hh, h) * e(-1, ky * ww, w)
                        xh[i, s, r, ky] = acc * scale
        for o in range(cout):
            for s in range(2):
                for r in range(mx):
                    kx = r if s == 0 else h - mx + r
                    for ky in range(my):
                        y = 0j
                        for i in range(cin):
                            y += xh[i, s, r, ky] * weight[s, r, ky, i, o]
                        c = 1.0 if (ky == 0 or 2 * ky == w) else 2.0
                        for hh in range(h):
                            for ww in range(w):
                                out[b, o, hh, ww] += c * (y * e(+1, kx * hh, h) * e(+1, ky * ww, w)).real
    return out * scale


def spectral_conv1d_loops(x, weight, modes: int):
    """The whole 1D operator as explicit loops (tiny inputs only)."""
    x = np.asarray(x, dtype=np.float64)
    weight = np.asarray(weight, dtype=np.complex128)
    b_n, cin, n = x.shape
    cout = weight.shape[-1]
    scale = 1.0 / math.sqrt(n)
    out = np.zeros((b_n, cout, n))
    for b in range(b_n):
        xh = np.zeros((cin, modes), dtype=np.complex128)
        for i in range(cin):
            for k in range(modes):
                acc = 0j
                for t in range(n):
                    ang = 2.0 * math.pi * ((k * t) % n) / n
                    acc += x[b, i, t] * complex(math.cos(ang), -math.sin(ang))
                xh[i, k] = acc * scale
        for o in range(cout):
            for k in range(modes):
                y = sum(xh[i, k] * weight[k, i, o] for i in range(cin))
                c = 1.0 if (k == 0 or 2 * k == n) else 2.0
                for t in range(n):
                    ang = 2.0 * math.pi * ((k * t) % n) / n
                    out[b, o, t] += c * (y * complex(math.cos(ang), math.sin(ang))).real
    return out * scale
