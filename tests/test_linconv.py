"""GPU parity of the zero-padded linear convolution (fno_linear_conv2d /
_1d and their weight-spectrum preparation) against the fp64 oracle's
direct definition, which the CPU suite pins against scipy / numpy
convolution and impulse shifts.  Same bar as the operator: relative L2
error <= 1e-5 and max-abs error <= 1e-4 * max|ref|.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import fft_spectral_convolution_amd as fno  # noqa: E402
import parity_log  # noqa: E402

pytestmark = pytest.mark.gpu

REL_L2 = 1e-5
MAX_ABS = 1e-4
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fno.lib()


def assert_close(gpu, ref, what):
    g = gpu.detach().cpu().numpy()
    g = g.astype(np.complex128) if np.iscomplexobj(g) else g.astype(np.float64)
    rel = np.linalg.norm((g - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    mx = np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300)
    print(f"  {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    parity_log.record(what, rel, mx)
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max-abs error {mx:.3e} > {MAX_ABS} * max|ref|"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


CASES_2D = [
    # B, Cin, Cout, H, W, kh, kw, crop (None: "same"), out size
    (2, 64, 64, 128, 128, 5, 5, None, None),          # the blog's 128x128, 64 -> 64, 5x5 case
    (2, 4, 6, 100, 100, 5, 5, None, None),            # non-power-of-two grid (padded to 128)
    (3, 3, 2, 7, 9, 3, 5, (0, 0), (9, 13)),           # the full convolution
    (1, 2, 3, 50, 30, 7, 4, (4, 1), (40, 20)),        # an arbitrary crop window
    (1, 2, 2, 300, 200, 9, 9, None, None),            # staged transforms (512 x 256)
    (2, 1, 1, 1, 33, 1, 4, None, None),               # single-row images
    (1, 2, 2, 6, 5000, 3, 3, None, None),             # rows padded beyond 4096 (5040 = 2^4 3^2 5 7)
]


@pytest.mark.parametrize("case", CASES_2D, ids=lambda c: "x".join(map(str, c[:7])))
def test_linear_conv2d(case):
    b, cin, cout, h, w, kh, kw, crop, size = case
    rng = np.random.default_rng(70)
    x = rng.uniform(-1, 1, (b, cin, h, w)).astype(np.float32)
    k = (rng.standard_normal((cout, cin, kh, kw)) / math.sqrt(cin * kh * kw)).astype(np.float32)
    ch, cw = crop if crop is not None else ((kh - 1) // 2, (kw - 1) // 2)
    ho, wo = size if size is not None else (h, w)
    out = fno.fno_linear_conv2d(dev(x), dev(k), crop=(ch, cw), out_size=(ho, wo))
    torch.cuda.synchronize()
    kernels = fno.fno_last_kernels()
    assert kernels[0] == "rows_fwd" and kernels[-1] == "rows_inv"      # padding and crop inside the row kernels
    ref = oracle.linear_conv2d_ref(x, k, ch, cw, ho, wo)
    assert_close(out, ref, f"linear conv {h}x{w} * {kh}x{kw}")


def test_linear_conv2d_weight_spectrum():
    # the prepared weight: sqrt(PH PW) * ortho R2C of the zero-padded kernels
    rng = np.random.default_rng(71)
    cout, cin, kh, kw, h, w = 3, 2, 3, 5, 12, 20
    k = rng.standard_normal((cout, cin, kh, kw)).astype(np.float32)
    ph, pw = fno.fno_linear_conv_length(h, kh), fno.fno_linear_conv_length(w, kw)
    assert (ph, pw) == (14, 24)           # the smallest even 7-smooth lengths >= 14 and 24
    wspec = fno.fno_linear_conv2d_prepare(dev(k), h, w)
    torch.cuda.synchronize()
    kp = np.zeros((cout, cin, ph, pw))
    kp[:, :, :kh, :kw] = k
    ref = math.sqrt(ph * pw) * np.transpose(oracle.forward_truncated_2d(kp, ph // 2, pw // 2 + 1), (2, 3, 4, 1, 0))
    assert_close(wspec, ref, "weight spectrum")


CASES_1D = [
    # B, Cin, Cout, N, K, crop (None: "same"), out length
    (4, 8, 8, 1000, 7, None, None),                   # non-power-of-two length (padded to 1024)
    (2, 3, 5, 2000, 64, 0, 2063),                     # the full convolution (padded to 4096)
    (3, 2, 2, 37, 5, 3, 30),                          # a crop window
    (2, 4, 4, 4096, 7, None, None),                   # the 4096-point sequences, 7 taps (padded to 4116)
]


@pytest.mark.parametrize("case", CASES_1D, ids=lambda c: "x".join(map(str, c[:5])))
def test_linear_conv1d(case):
    b, cin, cout, n, kk, crop, no = case
    if fno.fno_linear_conv_length(n, kk) == 0:
        pytest.skip("padded length beyond the transform range")
    rng = np.random.default_rng(72)
    x = rng.standard_normal((b, cin, n)).astype(np.float32)
    k = (rng.standard_normal((cout, cin, kk)) / math.sqrt(cin * kk)).astype(np.float32)
    c0 = crop if crop is not None else (kk - 1) // 2
    no = no if no is not None else n
    out = fno.fno_linear_conv1d(dev(x), dev(k), crop=c0, out_len=no)
    torch.cuda.synchronize()
    ref = oracle.linear_conv1d_ref(x, k, c0, no)
    assert_close(out, ref, f"linear conv1d {n} * {kk}")
