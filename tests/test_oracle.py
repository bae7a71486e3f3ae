"""Pins for the fp64 oracle (CPU only).

The oracle is trusted only because of these checks, each of which fixes the
answer from outside the oracle: closed forms of the transforms, Parseval,
identity / projector properties, the convolution theorem against a directly
computed circular convolution, a library FFT (numpy.fft) as an independent
witness, and brute-force loops on tiny inputs.  ``test_planted_mistakes``
plants plausible bugs into the oracle (a flipped sign, a conjugated weight,
a wrong block-1 index, a wrong C2R weight, transposed channels) and checks
that some pin catches each one.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import spectral as S

TRANSFORMS = ["dft", "fft"]


def rel(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    den = np.linalg.norm(b.ravel())
    return np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0)


def rand_c(rng, shape):
    return rng.standard_normal(shape) + 1j * rng.standard_normal(shape)


# --------------------------------------------------------------------------
# 1D transforms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64])
@pytest.mark.parametrize("sign", [-1, +1])
def test_dft_brute_vs_radix2(n, sign):
    rng = np.random.default_rng(n)
    a = rand_c(rng, (3, n))
    assert rel(S.fft_radix2(a, -1, sign), S.dft_brute(a, -1, sign)) < 1e-13


def test_dft_brute_vs_radix2_2d_8x8():
    rng = np.random.default_rng(7)
    a = rand_c(rng, (2, 8, 8))
    brute = S.dft_brute(S.dft_brute(a, 1, -1), 2, -1)
    fast = S.fft_radix2(S.fft_radix2(a, 2, -1), 1, -1)
    assert rel(fast, brute) < 1e-13


@pytest.mark.parametrize("n", [1, 4, 16, 32])
@pytest.mark.parametrize("fn", [S.dft_brute, S.fft_radix2])
def test_dft_impulse_constant_exponential(n, fn):
    delta = np.zeros(n)
    delta[0] = 1.0
    np.testing.assert_allclose(fn(delta), np.ones(n), atol=1e-13)
    np.testing.assert_allclose(fn(np.ones(n)), n * delta, atol=1e-12)
    # a single complex exponential e^{+2 pi i q t / n} lands in bin q with weight n
    q = 3 % n
    t = np.arange(n)
    e = np.exp(2j * np.pi * q * t / n)
    expect = np.zeros(n, dtype=complex)
    expect[q] = n
    np.testing.assert_allclose(fn(e), expect, atol=1e-11)


@pytest.mark.parametrize("n", [2, 8, 32, 128])
def test_transforms_vs_numpy_fft(n):
    rng = np.random.default_rng(n + 1)
    a = rand_c(rng, (4, n))
    ref = np.fft.fft(a, axis=-1)
    assert rel(S.dft_brute(a), ref) < 1e-13
    assert rel(S.fft_radix2(a), ref) < 1e-13
    assert rel(S.fft_radix2(a, sign=+1), np.fft.ifft(a, axis=-1) * n) < 1e-13


def test_radix2_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        S.fft_radix2(np.ones(6))


# --------------------------------------------------------------------------
# Forward transform + ortho scale
# --------------------------------------------------------------------------

def full_modes_xh_to_half(xh, h):
    """Map the full-modes truncated spectrum [.., 2, H/2, W/2+1] back to [.., H, W/2+1]."""
    mx = xh.shape[-2]
    assert 2 * mx == h
    return np.concatenate([xh[..., 0, :, :], xh[..., 1, :, :]], axis=-2)


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("h,w", [(8, 8), (16, 8), (4, 16)])
def test_forward_parseval(transform, h, w):
    rng = np.random.default_rng(h * 100 + w)
    x = rng.uniform(-1, 1, (2, 3, h, w))
    xh = S.forward_truncated_2d(x, h // 2, w // 2 + 1, transform)
    half = full_modes_xh_to_half(xh, h)
    c = np.full(w // 2 + 1, 2.0)
    c[0] = 1.0
    c[w // 2] = 1.0
    energy_x = np.sum(x ** 2, axis=(-2, -1))
    energy_k = np.sum(c * np.abs(half) ** 2, axis=(-2, -1))
    np.testing.assert_allclose(energy_k, energy_x, rtol=1e-13)


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("h,w,a,b", [(8, 8, 1, 2), (16, 8, 5, 3), (8, 16, 7, 1)])
def test_forward_single_cosine(transform, h, w, a, b):
    hh, ww = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    x = np.cos(2 * np.pi * (a * hh / h + b * ww / w))[None, None]
    half = full_modes_xh_to_half(S.forward_truncated_2d(x, h // 2, w // 2 + 1, transform), h)[0, 0]
    expect = np.zeros_like(half)
    expect[a, b] = math.sqrt(h * w) / 2
    np.testing.assert_allclose(half, expect, atol=1e-12)


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_forward_constant(transform):
    h, w = 16, 8
    x = np.ones((1, 1, h, w))
    half = full_modes_xh_to_half(S.forward_truncated_2d(x, h // 2, w // 2 + 1, transform), h)[0, 0]
    expect = np.zeros_like(half)
    expect[0, 0] = math.sqrt(h * w)
    np.testing.assert_allclose(half, expect, atol=1e-12)


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_forward_1d_closed_forms(transform):
    n = 32
    t = np.arange(n)
    x = np.cos(2 * np.pi * 5 * t / n)[None, None]
    xh = S.forward_truncated_1d(x, n // 2 + 1, transform)[0, 0]
    expect = np.zeros(n // 2 + 1, dtype=complex)
    expect[5] = math.sqrt(n) / 2
    np.testing.assert_allclose(xh, expect, atol=1e-12)


# --------------------------------------------------------------------------
# Truncation, kx mapping, mix and C2R closed forms
# --------------------------------------------------------------------------

def single_mode_weight(mx, my, s, r, ky, c):
    w = np.zeros((2, mx, my, 1, 1), dtype=complex)
    w[s, r, ky, 0, 0] = c
    return w


def inband_error(h, w, mx, my, a, b, c, transform="dft"):
    """|out - (Re c cos th - Im c sin th)| for x = cos th, th = 2 pi (a h/H + b w/W)."""
    hh, ww = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    th = 2 * np.pi * (a * hh / h + b * ww / w)
    x = np.cos(th)[None, None]
    if a < mx:
        s, r = 0, a
    else:
        s, r = 1, a - (h - mx)
    wt = single_mode_weight(mx, my, s, r, b, c)
    out = S.spectral_conv2d_ref(x, wt, mx, my, transform)[0, 0]
    expect = c.real * np.cos(th) - c.imag * np.sin(th)
    return np.max(np.abs(out - expect))


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("h,w,mx,my,a,b", [
    (16, 16, 4, 5, 3, 2),    # block 0, a = mx - 1
    (16, 16, 4, 5, 12, 2),   # block 1, r = 0 (kx = H - mx)
    (16, 16, 4, 5, 15, 4),   # block 1, r = mx - 1, ky = my - 1
    (32, 8, 3, 4, 1, 3),     # non-square
])
def test_inband_single_mode(transform, h, w, mx, my, a, b):
    assert inband_error(h, w, mx, my, a, b, 0.7 - 0.4j, transform) < 1e-12


def outband_max(h, w, mx, my, a, b, transform="dft"):
    hh, ww = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    x = np.cos(2 * np.pi * (a * hh / h + b * ww / w))[None, None]
    wt = np.ones((2, mx, my, 1, 1), dtype=complex) * (0.3 + 0.9j)
    return np.max(np.abs(S.spectral_conv2d_ref(x, wt, mx, my, transform)))


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("a,b", [(4, 2), (11, 2), (2, 5)])
def test_out_of_band_is_zero(transform, a, b):
    # H=W=16, mx=4, my=5: a=mx and a=H-mx-1 are dropped along H; b=my is dropped along W.
    assert outband_max(16, 16, 4, 5, a, b, transform) < 1e-12


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_two_corner_ky0(transform):
    h, w, mx, my, a = 16, 8, 5, 3, 2
    th = 2 * np.pi * a * np.arange(h) / h
    x = np.repeat(np.cos(th)[:, None], w, axis=1)[None, None]
    c1, c2 = 0.8 + 0.3j, -0.2 + 0.6j
    wt = np.zeros((2, mx, my, 1, 1), dtype=complex)
    wt[0, a, 0, 0, 0] = c1           # kx = a
    wt[1, mx - a, 0, 0, 0] = c2      # kx = H - mx + (mx - a) = H - a
    out = S.spectral_conv2d_ref(x, wt, mx, my, transform)[0, 0]
    expect = (c1 * np.exp(1j * th) + c2 * np.exp(-1j * th)).real / 2
    np.testing.assert_allclose(out, np.repeat(expect[:, None], w, axis=1), atol=1e-12)


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_dc_and_nyquist_imaginary_dropped(transform):
    h, w = 8, 8
    mx, my = 2, w // 2 + 1
    x = np.ones((1, 1, h, w))
    wt = single_mode_weight(mx, my, 0, 0, 0, 1j)
    assert np.max(np.abs(S.spectral_conv2d_ref(x, wt, mx, my, transform))) < 1e-12
    wt = single_mode_weight(mx, my, 0, 0, 0, 1.0)
    np.testing.assert_allclose(S.spectral_conv2d_ref(x, wt, mx, my, transform), x, atol=1e-12)
    # Nyquist column: x = (-1)^w sits entirely in ky = W/2 with weight c_{W/2} = 1
    alt = np.tile((-1.0) ** np.arange(w), (h, 1))[None, None]
    wt = single_mode_weight(mx, my, 0, 0, w // 2, 1j)
    assert np.max(np.abs(S.spectral_conv2d_ref(alt, wt, mx, my, transform))) < 1e-12
    wt = single_mode_weight(mx, my, 0, 0, w // 2, 1.0)
    np.testing.assert_allclose(S.spectral_conv2d_ref(alt, wt, mx, my, transform), alt, atol=1e-12)


# --------------------------------------------------------------------------
# Whole-operator invariants
# --------------------------------------------------------------------------

def identity_weight(mx, my, c):
    return np.broadcast_to(np.eye(c), (2, mx, my, c, c)).astype(complex)


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("h,w", [(8, 8), (16, 8), (4, 32), (2, 2)])
def test_identity_full_modes(transform, h, w):
    rng = np.random.default_rng(h + w)
    x = rng.uniform(-1, 1, (2, 3, h, w))
    out = S.spectral_conv2d_ref(x, identity_weight(h // 2, w // 2 + 1, 3), h // 2, w // 2 + 1, transform)
    np.testing.assert_allclose(out, x, atol=1e-13)


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("n", [2, 8, 64])
def test_identity_full_modes_1d(transform, n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((3, 2, n))
    wt = np.broadcast_to(np.eye(2), (n // 2 + 1, 2, 2)).astype(complex)
    np.testing.assert_allclose(S.spectral_conv1d_ref(x, wt, n // 2 + 1, transform), x, atol=1e-12)


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_projector_idempotent(transform):
    rng = np.random.default_rng(3)
    h, w, mx, my = 16, 16, 3, 4
    x = rng.uniform(-1, 1, (2, 2, h, w))
    wt = identity_weight(mx, my, 2).copy()
    # kx = H - mx at ky = 0 has no conjugate partner in the kept set (kx = mx is
    # dropped), so C2R keeps only half of it and the map is not idempotent there;
    # with that one mode switched off the operator is an orthogonal projector.
    wt[1, 0, 0] = 0.0
    once = S.spectral_conv2d_ref(x, wt, mx, my, transform)
    twice = S.spectral_conv2d_ref(once, wt, mx, my, transform)
    np.testing.assert_allclose(twice, once, atol=1e-13)
    assert rel(once, x) > 0.1      # it really projects


def circular_conv2d_direct(x, k):
    """out[b,o] = sum_i x[b,i] (*) k[i,o], circular, by explicit shifted sums."""
    b_n, cin, h, w = x.shape
    cout = k.shape[1]
    out = np.zeros((b_n, cout, h, w))
    for b in range(b_n):
        for o in range(cout):
            for i in range(cin):
                for hp in range(h):
                    for wp in range(w):
                        out[b, o] += x[b, i, hp, wp] * np.roll(k[i, o], (hp, wp), axis=(0, 1))
    return out


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("h,w", [(8, 8), (16, 8)])
def test_convolution_theorem_full_modes(transform, h, w):
    rng = np.random.default_rng(11)
    b_n, cin, cout = 2, 2, 3
    x = rng.uniform(-1, 1, (b_n, cin, h, w))
    k = rng.standard_normal((cin, cout, h, w))
    mx, my = h // 2, w // 2 + 1
    spec = np.fft.rfft2(k, axes=(-2, -1))                       # [Cin,Cout,H,W/2+1]
    kx = np.concatenate([np.arange(mx), h - mx + np.arange(mx)])
    wt = np.transpose(spec[:, :, kx, :my], (2, 3, 0, 1)).reshape(2, mx, my, cin, cout)
    out = S.spectral_conv2d_ref(x, wt, mx, my, transform)
    np.testing.assert_allclose(out, circular_conv2d_direct(x, k), atol=1e-11)


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_convolution_theorem_bandlimited_partial_modes(transform):
    rng = np.random.default_rng(12)
    h, w, mx, my = 16, 8, 3, 3
    b_n, cin, cout = 2, 2, 3
    x = rng.uniform(-1, 1, (b_n, cin, h, w))
    spec = np.zeros((cin, cout, h, w // 2 + 1), dtype=complex)
    kx = np.concatenate([np.arange(mx), h - mx + np.arange(mx)])
    for q in kx:
        spec[:, :, q, :my] = rand_c(rng, (cin, cout, my))
    # Hermitian consistency of the ky = 0 column over the kept kx set
    spec[:, :, 0, 0] = spec[:, :, 0, 0].real
    for r in range(1, mx):
        spec[:, :, h - r, 0] = np.conj(spec[:, :, r, 0])
    spec[:, :, h - mx, 0] = 0.0           # its partner kx = mx is not kept
    k = np.fft.irfft2(spec, s=(h, w), axes=(-2, -1))
    np.testing.assert_allclose(np.fft.rfft2(k, axes=(-2, -1)), spec, atol=1e-12)
    wt = np.transpose(spec[:, :, kx, :my], (2, 3, 0, 1)).reshape(2, mx, my, cin, cout)
    out = S.spectral_conv2d_ref(x, wt, mx, my, transform)
    np.testing.assert_allclose(out, circular_conv2d_direct(x, k), atol=1e-11)


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_convolution_theorem_1d(transform):
    rng = np.random.default_rng(13)
    n, b_n, cin, cout = 16, 3, 2, 3
    x = rng.standard_normal((b_n, cin, n))
    k = rng.standard_normal((cin, cout, n))
    spec = np.fft.rfft(k, axis=-1)                                 # [Cin,Cout,N/2+1]
    wt = np.transpose(spec, (2, 0, 1))
    out = S.spectral_conv1d_ref(x, wt, n // 2 + 1, transform)
    direct = np.zeros((b_n, cout, n))
    for b in range(b_n):
        for o in range(cout):
            for i in range(cin):
                for t in range(n):
                    direct[b, o] += x[b, i, t] * np.roll(k[i, o], t)
    np.testing.assert_allclose(out, direct, atol=1e-11)


@pytest.mark.parametrize("transform", TRANSFORMS)
def test_linearity(transform):
    rng = np.random.default_rng(5)
    h, w, mx, my = 16, 8, 3, 4
    x1 = rng.uniform(-1, 1, (2, 3, h, w))
    x2 = rng.uniform(-1, 1, (2, 3, h, w))
    w1 = rand_c(rng, (2, mx, my, 3, 2))
    w2 = rand_c(rng, (2, mx, my, 3, 2))
    f = lambda x, wt: S.spectral_conv2d_ref(x, wt, mx, my, transform)
    np.testing.assert_allclose(f(0.3 * x1 - 1.7 * x2, w1), 0.3 * f(x1, w1) - 1.7 * f(x2, w1), atol=1e-12)
    np.testing.assert_allclose(f(x1, 0.3 * w1 + 2.0 * w2), 0.3 * f(x1, w1) + 2.0 * f(x1, w2), atol=1e-12)


def test_mode_tagging():
    rng = np.random.default_rng(6)
    h, w, mx, my = 8, 8, 2, 3
    x = rng.uniform(-1, 1, (1, 2, h, w))
    wt = rand_c(rng, (2, mx, my, 2, 2))
    full = S.spectral_conv2d_ref(x, wt, mx, my)
    acc = np.zeros_like(full)
    for s in range(2):
        for r in range(mx):
            for ky in range(my):
                tag = np.zeros_like(wt)
                tag[s, r, ky] = wt[s, r, ky]
                part = S.spectral_conv2d_ref(x, tag, mx, my)
                assert np.max(np.abs(part)) > 0
                acc += part
    np.testing.assert_allclose(acc, full, atol=1e-13)


def test_channel_permutation():
    rng = np.random.default_rng(8)
    h, w, mx, my, c = 8, 16, 2, 5, 4
    x = rng.uniform(-1, 1, (2, c, h, w))
    sigma = [2, 0, 3, 1]
    wt = np.zeros((2, mx, my, c, c), dtype=complex)
    for o in range(c):
        wt[..., sigma[o], o] = 1.0
    out = S.spectral_conv2d_ref(x, wt, mx, my)
    one = np.ones((2, mx, my, 1, 1), dtype=complex)
    for o in range(c):
        proj = S.spectral_conv2d_ref(x[:, sigma[o]:sigma[o] + 1], one, mx, my)[:, 0]
        np.testing.assert_allclose(out[:, o], proj, atol=1e-13)


# --------------------------------------------------------------------------
# The two transform paths and the loop twins
# --------------------------------------------------------------------------

@pytest.mark.parametrize("h,w,mx,my", [(32, 32, 8, 8), (16, 64, 5, 33), (64, 8, 32, 2)])
def test_dft_and_fft_paths_agree(h, w, mx, my):
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (2, 3, h, w)).astype(np.float32)
    wt = (rand_c(rng, (2, mx, my, 3, 2)) / 6).astype(np.complex64)
    a, xa, ya = S.spectral_conv2d_ref(x, wt, mx, my, "dft", return_stages=True)
    b, xb, yb = S.spectral_conv2d_ref(x, wt, mx, my, "fft", return_stages=True)
    assert rel(xa, xb) < 1e-13
    assert rel(ya, yb) < 1e-13
    assert rel(a, b) < 1e-13


def test_1d_dft_and_fft_paths_agree():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3, 4, 256))
    wt = rand_c(rng, (20, 4, 5))
    assert rel(S.spectral_conv1d_ref(x, wt, 20, "dft"), S.spectral_conv1d_ref(x, wt, 20, "fft")) < 1e-13


@pytest.mark.parametrize("h,w,mx,my", [(4, 4, 1, 2), (8, 4, 2, 3), (4, 8, 2, 5)])
def test_loops_twin_2d(h, w, mx, my):
    rng = np.random.default_rng(h * w)
    x = rng.uniform(-1, 1, (2, 2, h, w))
    wt = rand_c(rng, (2, mx, my, 2, 3))
    np.testing.assert_allclose(S.spectral_conv2d_ref(x, wt, mx, my),
                               S.spectral_conv2d_loops(x, wt, mx, my), atol=1e-12)


def test_loops_twin_1d():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 16))
    wt = rand_c(rng, (9, 3, 2))
    np.testing.assert_allclose(S.spectral_conv1d_ref(x, wt, 9), S.spectral_conv1d_loops(x, wt, 9), atol=1e-12)


def test_shape_checks():
    x = np.zeros((1, 1, 8, 8))
    with pytest.raises(ValueError):
        S.spectral_conv2d_ref(x, np.zeros((2, 5, 2, 1, 1)), 5, 2)     # 2*mx > H
    with pytest.raises(ValueError):
        S.spectral_conv2d_ref(x, np.zeros((2, 2, 6, 1, 1)), 2, 6)     # my > W/2+1


# --------------------------------------------------------------------------
# Planted mistakes: each one must be caught by at least one pin above
# --------------------------------------------------------------------------

def _pins_pass():
    """Run a compact set of pins against the (possibly mutated) oracle."""
    checks = []
    checks.append(inband_error(16, 16, 4, 5, 3, 2, 0.7 - 0.4j) < 1e-12)
    checks.append(inband_error(16, 16, 4, 5, 12, 2, 0.7 - 0.4j) < 1e-12)
    rng = np.random.default_rng(0)
    x = rng.uniform(-1, 1, (1, 2, 8, 8))
    out = S.spectral_conv2d_ref(x, identity_weight(4, 5, 2), 4, 5)
    checks.append(np.max(np.abs(out - x)) < 1e-12)
    xo = np.ones((1, 1, 8, 8))
    checks.append(np.max(np.abs(S.spectral_conv2d_ref(xo, single_mode_weight(2, 5, 0, 0, 0, 1j), 2, 5))) < 1e-12)
    # convolution theorem with a non-symmetric channel coupling
    h = w = 8
    x = rng.uniform(-1, 1, (1, 3, h, w))
    k = rng.standard_normal((3, 3, h, w))
    spec = np.fft.rfft2(k, axes=(-2, -1))
    kx = np.concatenate([np.arange(4), 4 + np.arange(4)])
    wt = np.transpose(spec[:, :, kx, :5], (2, 3, 0, 1)).reshape(2, 4, 5, 3, 3)
    checks.append(np.max(np.abs(S.spectral_conv2d_ref(x, wt, 4, 5) - circular_conv2d_direct(x, k))) < 1e-10)
    return all(checks)


def test_pins_pass_on_clean_oracle():
    assert _pins_pass()


def test_planted_mistakes(monkeypatch):
    import contextlib

    mutations = []

    def flip_forward_sign(n, rows, cols, sign, _orig=S.dft_matrix):
        return _orig(n, rows, cols, -sign)
    mutations.append(("dft_matrix", flip_forward_sign))

    def conj_mix(xh, weight, _orig=S.mix_2d):
        return _orig(xh, np.conj(weight))
    mutations.append(("mix_2d", conj_mix))

    def transposed_mix(xh, weight):
        return np.einsum("bisrk,srkoi->bosrk", np.asarray(xh, complex), np.asarray(weight, complex))
    mutations.append(("mix_2d", transposed_mix))

    def shifted_block1(h, mx, _orig=S.kept_kx):
        k = _orig(h, mx).copy()
        k[mx:] = (k[mx:] + 1) % h
        return k
    mutations.append(("kept_kx", shifted_block1))

    def all_twos(w, my):
        return np.full(my, 2.0)
    mutations.append(("c2r_weights", all_twos))

    for name, fn in mutations:
        with monkeypatch.context() as m:
            m.setattr(S, name, fn)
            try:
                caught = not _pins_pass()
            except Exception:
                caught = True
        assert caught, f"planted mistake in {name} ({fn.__name__}) was not caught"


# --------------------------------------------------------------------------
# Gradients: the adjoint identity <A x, g> = <x, A^T g> and the exact change
# of the (linear-in-W) loss under a weight perturbation
# --------------------------------------------------------------------------

BWD_2D = [(2, 3, 4, 8, 8, 2, 3), (1, 2, 3, 16, 8, 3, 5), (2, 2, 2, 8, 16, 4, 9), (1, 1, 2, 4, 4, 2, 3)]


def _loss_2d(x, w, g, mx, my, transform="dft"):
    return float(np.sum(g * S.spectral_conv2d_ref(x, w, mx, my, transform)))


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("shape", BWD_2D)
def test_backward_adjoint_2d(transform, shape):
    b, cin, cout, h, w, mx, my = shape
    rng = np.random.default_rng(31)
    x = rng.standard_normal((b, cin, h, w))
    wt = rand_c(rng, (2, mx, my, cin, cout))
    g = rng.standard_normal((b, cout, h, w))
    gx, _ = S.spectral_conv2d_backward_ref(x, wt, g, mx, my, transform)
    lhs = _loss_2d(x, wt, g, mx, my, transform)          # <A x, g>
    rhs = float(np.sum(x * gx))                           # <x, A^T g>
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("shape", BWD_2D)
def test_backward_weight_exact_difference_2d(transform, shape):
    # L is linear in W: L(W + E) - L(W) = Re sum conj(dL/dW) E exactly
    b, cin, cout, h, w, mx, my = shape
    rng = np.random.default_rng(32)
    x = rng.standard_normal((b, cin, h, w))
    wt = rand_c(rng, (2, mx, my, cin, cout))
    g = rng.standard_normal((b, cout, h, w))
    e = rand_c(rng, wt.shape)
    _, gw = S.spectral_conv2d_backward_ref(x, wt, g, mx, my, transform)
    diff = _loss_2d(x, wt + e, g, mx, my, transform) - _loss_2d(x, wt, g, mx, my, transform)
    pred = float(np.real(np.sum(np.conj(gw) * e)))
    assert abs(diff - pred) <= 1e-10 * max(1.0, abs(diff))
    # and one coordinate at a time, real and imaginary directions separately
    for idx in [(0, 0, 0, 0, 0), (1, mx - 1, my - 1, cin - 1, cout - 1), (0, 0, my - 1, 0, cout - 1)]:
        for unit, part in ((1.0, np.real), (1j, np.imag)):
            e1 = np.zeros_like(wt)
            e1[idx] = unit
            d1 = _loss_2d(x, wt + e1, g, mx, my, transform) - _loss_2d(x, wt, g, mx, my, transform)
            assert abs(d1 - part(gw[idx])) <= 1e-10 * max(1.0, abs(d1))


def test_backward_ones_weight_full_modes_is_identity_adjoint():
    # full modes, identity weights: the operator is the identity, so its
    # adjoint returns g itself
    rng = np.random.default_rng(33)
    h, w, c = 8, 8, 3
    mx, my = h // 2, w // 2 + 1
    wt = np.zeros((2, mx, my, c, c), dtype=np.complex128)
    for i in range(c):
        wt[..., i, i] = 1.0
    g = rng.standard_normal((2, c, h, w))
    gx, _ = S.spectral_conv2d_backward_ref(rng.standard_normal((2, c, h, w)), wt, g, mx, my)
    assert rel(gx, g) < 1e-12


BWD_1D = [(2, 3, 4, 16, 5), (1, 2, 2, 8, 5), (3, 1, 2, 32, 1)]


def _loss_1d(x, w, g, modes, transform="dft"):
    return float(np.sum(g * S.spectral_conv1d_ref(x, w, modes, transform)))


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("shape", BWD_1D)
def test_backward_1d(transform, shape):
    b, cin, cout, n, modes = shape
    rng = np.random.default_rng(34)
    x = rng.standard_normal((b, cin, n))
    wt = rand_c(rng, (modes, cin, cout))
    g = rng.standard_normal((b, cout, n))
    gx, gw = S.spectral_conv1d_backward_ref(x, wt, g, modes, transform)
    lhs = _loss_1d(x, wt, g, modes, transform)
    assert abs(lhs - float(np.sum(x * gx))) <= 1e-11 * max(1.0, abs(lhs))
    e = rand_c(rng, wt.shape)
    diff = _loss_1d(x, wt + e, g, modes, transform) - lhs
    assert abs(diff - float(np.real(np.sum(np.conj(gw) * e)))) <= 1e-10 * max(1.0, abs(diff))


def test_backward_planted_mistakes():
    # plausible slips in the gradient formulas, each caught by the pins above
    b, cin, cout, h, w, mx, my = 2, 3, 4, 8, 8, 2, 5     # my = W/2 + 1: Nyquist column kept
    rng = np.random.default_rng(35)
    x = rng.standard_normal((b, cin, h, w))
    wt = rand_c(rng, (2, mx, my, cin, cout))
    g = rng.standard_normal((b, cout, h, w))
    e = rand_c(rng, wt.shape)
    gx, gw = S.spectral_conv2d_backward_ref(x, wt, g, mx, my)
    lhs = _loss_2d(x, wt, g, mx, my)
    diff = _loss_2d(x, wt + e, g, mx, my) - lhs

    def adjoint_ok(gx_try):
        return abs(lhs - float(np.sum(x * gx_try))) <= 1e-11 * max(1.0, abs(lhs))

    def weight_ok(gw_try):
        return abs(diff - float(np.real(np.sum(np.conj(gw_try) * e)))) <= 1e-10 * max(1.0, abs(diff))

    assert adjoint_ok(gx) and weight_ok(gw)
    gh = S.forward_truncated_2d(g, mx, my)
    xh = S.forward_truncated_2d(x, mx, my)
    c = S.c2r_weights(w, my)[None, None, :, None, None]
    # weight not conjugated in the input gradient
    assert not adjoint_ok(S.inverse_from_truncated_2d(np.einsum("bosrk,srkio->bisrk", gh, wt), h, w))
    # C2R weights applied to the input gradient as well
    assert not adjoint_ok(S.inverse_from_truncated_2d(
        np.einsum("bosrk,srkio->bisrk", gh, np.conj(wt)) * S.c2r_weights(w, my), h, w))
    # C2R weights missing from the weight gradient
    assert not weight_ok(np.einsum("bisrk,bosrk->srkio", np.conj(xh), gh))
    # conjugate on the wrong factor
    assert not weight_ok(np.einsum("bisrk,bosrk->srkio", xh, np.conj(gh)) * c)
    # batch not summed (first item only)
    assert not weight_ok(np.einsum("isrk,osrk->srkio", np.conj(xh[0]), gh[0]) * c)


# --------------------------------------------------------------------------
# Fused layer tail: gelu(conv + bias + branch) or gelu(conv + bias) + branch
# --------------------------------------------------------------------------

# standard normal CDF Phi(u) from a printed table (to double precision)
PHI_TABLE = {
    -2.0: 0.022750131948179195,
    -1.0: 0.15865525393145707,
    -0.5: 0.3085375387259869,
    0.0: 0.5,
    0.5: 0.6914624612740131,
    1.0: 0.8413447460685429,
    2.0: 0.9772498680518208,
    3.0: 0.9986501019683699,
}


def test_gelu_against_normal_cdf_table():
    for u, phi in PHI_TABLE.items():
        assert abs(float(S.gelu(u)) - u * phi) <= 1e-15 * max(1.0, abs(u))
    # the tanh approximation of GELU would miss the table by ~1.5e-4 at u = 1
    u = 1.0
    tanh_form = 0.5 * u * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))
    assert abs(tanh_form - u * PHI_TABLE[1.0]) > 1e-4


def test_gelu_odd_part_and_tails():
    # Phi(u) + Phi(-u) = 1  =>  gelu(u) - gelu(-u) = u
    u = np.random.default_rng(40).standard_normal(1000) * 3
    assert np.max(np.abs(S.gelu(u) - S.gelu(-u) - u)) <= 1e-14
    assert abs(float(S.gelu(12.0)) - 12.0) <= 1e-14 and abs(float(S.gelu(-12.0))) <= 1e-14


def _dc_identity_weight(rng, shape, c):
    # random weights, except the DC mode of block 0, which is the real identity
    wt = rand_c(rng, shape)
    wt[(0,) * (len(shape) - 2)] = np.eye(c)
    return wt


TABLE_POINTS = np.array(sorted(PHI_TABLE))


@pytest.mark.parametrize("branch_after", [False, True])
def test_layer_tail_closed_form_2d(branch_after):
    # x constant per (b, i): only the DC mode is non-zero, so with the
    # identity DC weight conv[b, o] = x[b, o] at every pixel, and the layer
    # output is a table value of gelu wherever its argument is a table point
    b, c, h, w, mx, my = 3, 3, 8, 16, 2, 3
    rng = np.random.default_rng(41)
    target = rng.choice(TABLE_POINTS, size=(b, c))
    const = rng.standard_normal((b, c))
    bias = rng.standard_normal(c)
    if branch_after:
        const = target - bias[None, :]               # gelu argument = target
        d = rng.standard_normal((b, c))
    else:
        d = target - const - bias[None, :]
    x = np.broadcast_to(const[:, :, None, None], (b, c, h, w)).copy()
    branch = np.broadcast_to(d[:, :, None, None], (b, c, h, w)).copy()
    wt = _dc_identity_weight(rng, (2, mx, my, c, c), c)
    out = S.spectral_conv2d_gelu_ref(x, wt, mx, my, bias=bias, branch=branch, branch_after=branch_after)
    phi = np.vectorize(PHI_TABLE.get)(target)
    expect = target * phi + (d if branch_after else 0.0)
    assert np.max(np.abs(out - expect[:, :, None, None])) <= 1e-12
    # planted mistakes, each off the table
    conv = S.spectral_conv2d_ref(x, wt, mx, my)
    wrong = {
        "bias along the batch axis": S.gelu(conv + bias[:, None, None, None] + (0 if branch_after else branch))
        + (branch if branch_after else 0),
        "branch on the other side of the activation": (S.gelu(conv + bias[None, :, None, None]) + branch)
        if not branch_after else S.gelu(conv + bias[None, :, None, None] + branch),
        "bias after the activation": S.gelu(conv + (0 if branch_after else branch)) + bias[None, :, None, None]
        + (branch if branch_after else 0),
    }
    for name, val in wrong.items():
        assert np.max(np.abs(val - expect[:, :, None, None])) > 1e-3, name


@pytest.mark.parametrize("branch_after", [False, True])
def test_layer_tail_closed_form_1d(branch_after):
    b, c, n, modes = 2, 4, 16, 5
    rng = np.random.default_rng(42)
    target = rng.choice(TABLE_POINTS, size=(b, c))
    bias = rng.standard_normal(c)
    d = rng.standard_normal((b, c))
    const = target - bias[None, :] - (0.0 if branch_after else d)
    x = np.broadcast_to(const[:, :, None], (b, c, n)).copy()
    branch = np.broadcast_to(d[:, :, None], (b, c, n)).copy()
    wt = _dc_identity_weight(rng, (modes, c, c), c)
    out = S.spectral_conv1d_gelu_ref(x, wt, modes, bias=bias, branch=branch, branch_after=branch_after)
    expect = target * np.vectorize(PHI_TABLE.get)(target) + (d if branch_after else 0.0)
    assert np.max(np.abs(out - expect[:, :, None])) <= 1e-12


def test_layer_tail_optional_terms():
    # no bias and no branch: gelu of the plain operator; the two orders agree
    rng = np.random.default_rng(43)
    x = rng.standard_normal((2, 3, 8, 8))
    wt = rand_c(rng, (2, 2, 3, 3, 4))
    conv = S.spectral_conv2d_ref(x, wt, 2, 3)
    for after in (False, True):
        out = S.spectral_conv2d_gelu_ref(x, wt, 2, 3, branch_after=after)
        assert np.max(np.abs(out - S.gelu(conv))) == 0.0


# --------------------------------------------------------------------------
# Diagonal global filter: one complex weight per kept mode and channel
# --------------------------------------------------------------------------

def _diag_weight(mask):
    # mask [..., C] -> weight [..., C, C] with the mask on the diagonal
    c = mask.shape[-1]
    wt = np.zeros(mask.shape + (c,), dtype=np.complex128)
    for i in range(c):
        wt[..., i, i] = mask[..., i]
    return wt


@pytest.mark.parametrize("transform", TRANSFORMS)
@pytest.mark.parametrize("shape", [(2, 3, 8, 8, 2, 3), (1, 4, 16, 8, 8, 5), (2, 2, 8, 16, 3, 9)])
def test_filter_is_conv_with_diagonal_weight(transform, shape):
    # the filter equals the (independently pinned) spectral convolution whose
    # weight is diagonal in the channels
    b, c, h, w, mx, my = shape
    rng = np.random.default_rng(50)
    x = rng.standard_normal((b, c, h, w))
    mask = rand_c(rng, (2, mx, my, c))
    out = S.spectral_filter2d_ref(x, mask, mx, my, transform)
    assert rel(out, S.spectral_conv2d_ref(x, _diag_weight(mask), mx, my, transform)) < 1e-12
    x1 = rng.standard_normal((b, c, w))
    m1 = rand_c(rng, (my, c))
    out1 = S.spectral_filter1d_ref(x1, m1, my, transform)
    assert rel(out1, S.spectral_conv1d_ref(x1, _diag_weight(m1), my, transform)) < 1e-12


def test_filter_full_modes_unit_mask_is_identity():
    rng = np.random.default_rng(51)
    h, w, c = 8, 16, 3
    x = rng.standard_normal((2, c, h, w))
    out = S.spectral_filter2d_ref(x, np.ones((2, h // 2, w // 2 + 1, c)), h // 2, w // 2 + 1)
    assert rel(out, x) < 1e-12
    x1 = rng.standard_normal((2, c, w))
    assert rel(S.spectral_filter1d_ref(x1, np.ones((w // 2 + 1, c)), w // 2 + 1), x1) < 1e-12


@pytest.mark.parametrize("block", [0, 1])
def test_filter_single_cosine_closed_form(block):
    # x = cos(theta), theta = 2 pi (kx h / H + ky w / W), 0 < ky < W/2, with kx
    # in block 0 (kx = r) or block 1 (kx = H - mx + r): the kept half spectrum
    # holds sqrt(HW)/2 at (kx, ky) only, so the output is Re(m e^{i theta})
    # = a cos(theta) - b sin(theta) for the mask value m = a + ib there
    h, w, mx, my, c = 16, 16, 4, 5, 2
    r, ky = 2, 3
    kx = r if block == 0 else h - mx + r
    hh, ww = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    theta = 2 * np.pi * (kx * hh / h + ky * ww / w)
    x = np.broadcast_to(np.cos(theta), (1, c, h, w)).copy()
    mask = np.zeros((2, mx, my, c), dtype=np.complex128)
    vals = [0.7 - 1.3j, -0.4 + 0.25j]
    for ch in range(c):
        mask[block, r, ky, ch] = vals[ch]
    out = S.spectral_filter2d_ref(x, mask, mx, my)
    for ch in range(c):
        a, b = vals[ch].real, vals[ch].imag
        assert np.max(np.abs(out[0, ch] - (a * np.cos(theta) - b * np.sin(theta)))) < 1e-12
    # planted mistakes: a conjugated mask, the channels of the mask swapped
    conj = S.spectral_filter2d_ref(x, np.conj(mask), mx, my)
    swapped = S.spectral_filter2d_ref(x, mask[..., ::-1], mx, my)
    expect0 = vals[0].real * np.cos(theta) - vals[0].imag * np.sin(theta)
    assert np.max(np.abs(conj[0, 0] - expect0)) > 0.1
    assert np.max(np.abs(swapped[0, 0] - expect0)) > 0.1


def test_filter_1d_single_cosine_closed_form():
    n, modes, c, k = 32, 6, 3, 4
    t = np.arange(n)
    theta = 2 * np.pi * k * t / n
    x = np.broadcast_to(np.cos(theta), (2, c, n)).copy()
    mask = np.zeros((modes, c), dtype=np.complex128)
    mask[k] = [1.5 + 0.5j, -2.0j, 0.3]
    out = S.spectral_filter1d_ref(x, mask, modes)
    for ch in range(c):
        m = mask[k, ch]
        assert np.max(np.abs(out[:, ch] - (m.real * np.cos(theta) - m.imag * np.sin(theta)))) < 1e-12


# --------------------------------------------------------------------------
# Linear (zero-padded) convolution
# --------------------------------------------------------------------------

def test_linear_conv_against_library_convolution():
    from scipy.signal import convolve
    rng = np.random.default_rng(60)
    x = rng.standard_normal((2, 3, 7, 9))
    k = rng.standard_normal((4, 3, 3, 5))
    y = S.linear_conv2d_ref(x, k)
    assert y.shape == (2, 4, 9, 13)
    for b in range(2):
        for o in range(4):
            ref = sum(convolve(x[b, i], k[o, i], mode="full") for i in range(3))
            assert np.max(np.abs(y[b, o] - ref)) < 1e-12
    x1 = rng.standard_normal((2, 2, 11))
    k1 = rng.standard_normal((3, 2, 4))
    y1 = S.linear_conv1d_ref(x1, k1)
    for b in range(2):
        for o in range(3):
            ref = sum(np.convolve(x1[b, i], k1[o, i]) for i in range(2))
            assert np.max(np.abs(y1[b, o] - ref)) < 1e-12


def test_linear_conv_delta_kernel_and_crop():
    # a unit impulse at (dh, dw) shifts x by (dh, dw); the 'same' crop of a
    # centred impulse returns x itself
    rng = np.random.default_rng(61)
    x = rng.standard_normal((1, 2, 6, 8))
    k = np.zeros((2, 2, 5, 3))
    k[0, 0, 2, 1] = 1.0
    k[1, 1, 2, 1] = 1.0
    same = S.linear_conv2d_ref(x, k, 2, 1, 6, 8)
    assert np.max(np.abs(same - x)) == 0.0
    k2 = np.zeros((1, 2, 5, 3))
    k2[0, 1, 4, 0] = 1.0
    full = S.linear_conv2d_ref(x, k2)
    assert np.max(np.abs(full[0, 0, 4:10, 0:8] - x[0, 1])) == 0.0
    assert np.count_nonzero(full) == np.count_nonzero(x[0, 1])      # nothing lands elsewhere


def test_linear_conv_through_padded_spectral_conv():
    # the method the GPU path uses: zero-pad both operands to a power-of-two
    # grid P >= N + k - 1, spectral convolution at full modes with
    # W = sqrt(PH PW) * ortho-R2C(kernel), crop; equal to the definition
    rng = np.random.default_rng(62)
    b, cin, cout, h, w, kh, kw = 2, 3, 2, 6, 5, 3, 4
    x = rng.standard_normal((b, cin, h, w))
    k = rng.standard_normal((cout, cin, kh, kw))
    ph, pw = 8, 8
    xp = np.zeros((b, cin, ph, pw))
    xp[:, :, :h, :w] = x
    kp = np.zeros((cout, cin, ph, pw))
    kp[:, :, :kh, :kw] = k
    mx, my = ph // 2, pw // 2 + 1
    kh_spec = S.forward_truncated_2d(kp, mx, my)                     # [Cout,Cin,2,mx,my]
    wt = math.sqrt(ph * pw) * np.transpose(kh_spec, (2, 3, 4, 1, 0))  # [2,mx,my,Cin,Cout]
    y = S.spectral_conv2d_ref(xp, wt, mx, my)
    ref = S.linear_conv2d_ref(x, k)
    assert np.max(np.abs(y[:, :, :h + kh - 1, :w + kw - 1] - ref)) < 1e-12
    # planted mistake: without the sqrt(PH PW) factor the result is off
    y_bad = S.spectral_conv2d_ref(xp, wt / math.sqrt(ph * pw), mx, my)
    assert np.max(np.abs(y_bad[:, :, :h + kh - 1, :w + kw - 1] - ref)) > 0.1


# --------------------------------------------------------------------------
# Lengths that are not powers of two (the definition holds for any length)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [3, 5, 6, 7, 12, 15, 45, 100])
def test_dft_brute_vs_numpy_fft_any_length(n):
    a = np.random.default_rng(80 + n).standard_normal((2, n)) + 1j * np.random.default_rng(90 + n).standard_normal((2, n))
    assert rel(S.dft_brute(a, sign=-1), np.fft.fft(a, axis=-1)) < 1e-13
    assert rel(S.dft_brute(a, sign=+1), np.fft.ifft(a, axis=-1) * n) < 1e-13


@pytest.mark.parametrize("h,w", [(6, 10), (6, 9), (12, 15)])
def test_convolution_theorem_full_modes_any_length(h, w):
    # even H (every kx kept by 2 mx = H); W odd or even (the half spectrum
    # W//2 + 1 has no Nyquist bin when W is odd)
    rng = np.random.default_rng(81)
    b_n, cin, cout = 2, 2, 3
    x = rng.uniform(-1, 1, (b_n, cin, h, w))
    k = rng.standard_normal((cin, cout, h, w))
    mx, my = h // 2, w // 2 + 1
    spec = np.fft.rfft2(k, axes=(-2, -1))
    kx = np.concatenate([np.arange(mx), h - mx + np.arange(mx)])
    wt = np.transpose(spec[:, :, kx, :my], (2, 3, 0, 1)).reshape(2, mx, my, cin, cout)
    out = S.spectral_conv2d_ref(x, wt, mx, my)
    np.testing.assert_allclose(out, circular_conv2d_direct(x, k), atol=1e-11)


@pytest.mark.parametrize("n", [9, 15, 20])
def test_identity_full_modes_1d_any_length(n):
    rng = np.random.default_rng(82)
    x = rng.standard_normal((2, 3, n))
    wt = np.broadcast_to(np.eye(3, dtype=np.complex128), (n // 2 + 1, 3, 3)).copy()
    assert rel(S.spectral_conv1d_ref(x, wt, n // 2 + 1), x) < 1e-12
