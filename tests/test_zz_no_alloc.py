"""The entry point that allocates nothing (fno_spectral_conv2d_noalloc),
called through the C ABI, against fno_spectral_conv2d on the same inputs: two
calls in a row, the second with a smaller input, each to the parity bar
(relative L2 <= 1e-5, max-abs <= 1e-4 * max|ref|; both run the same kernels,
so the results are expected to be equal).  Also: a shape whose spectra need
more than the fixed array is refused with FNO_ERR_TOO_LARGE, a length that is
not a power of two with FNO_ERR_SHAPE.  fno_init runs first, so the test
passes in a fresh process as well as after the other tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import fft_spectral_convolution_amd as fno  # noqa: E402
from fft_spectral_convolution_amd.inputs import Config, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fno.lib()
    fno.fno_init()


def _close(got, ref, what):
    g = got.double().cpu().numpy()
    r = ref.double().cpu().numpy()
    rel = np.linalg.norm((g - r).ravel()) / np.linalg.norm(r.ravel())
    mx = np.max(np.abs(g - r)) / np.max(np.abs(r))
    print(f"  {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    assert rel <= 1e-5 and mx <= 1e-4, what


def _pair(cfg, seed):
    x, w = make_inputs(cfg, seed)
    xd, wd = torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV)
    out = torch.full((cfg.B, cfg.Cout, cfg.H, cfg.W), float("nan"), device=DEV)
    fno.fno_spectral_conv2d_noalloc(xd, wd, cfg.mx, cfg.my, out=out)
    ref = fno.fno_spectral_conv2d(xd, wd, cfg.mx, cfg.my)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_matches_plain_call_twice():
    # the 128x128 workload (its spectra fill the 64 MiB array exactly), then
    # a smaller grid whose call reuses the array's first part
    big = Config("na_big", "2d", 32, 64, 64, 128, 128, 32, 32, "uniform")
    small = Config("na_small", "2d", 3, 8, 12, 64, 64, 16, 16, "uniform")
    out, ref = _pair(big, 0)
    _close(out, ref, "noalloc 128x128 B=32 64->64")
    assert torch.equal(out, ref)
    out, ref = _pair(small, 1)
    _close(out, ref, "noalloc 64x64 B=3 8->12")
    assert torch.equal(out, ref)


def test_noalloc_staged_schedule():
    # a tall grid: row spectrum plus both truncated spectra in the array
    cfg = Config("na_tall", "2d", 1, 4, 4, 1024, 256, 16, 16, "uniform")
    out, ref = _pair(cfg, 2)
    _close(out, ref, "noalloc 1024x256 staged")
    assert torch.equal(out, ref)


def test_noalloc_refuses_what_it_cannot_hold():
    limit = fno.fno_noalloc_scratch_bytes()
    assert limit == 64 << 20
    x = torch.zeros((33, 64, 128, 128), device=DEV)       # one batch item more than fits
    w = torch.zeros((2, 32, 32, 64, 64), dtype=torch.complex64, device=DEV)
    with pytest.raises(fno.FnoError) as ei:
        fno.fno_spectral_conv2d_noalloc(x, w, 32, 32)
    assert ei.value.status == -10
    x = torch.zeros((1, 2, 96, 96), device=DEV)            # not a power of two
    w = torch.zeros((2, 8, 8, 2, 2), dtype=torch.complex64, device=DEV)
    with pytest.raises(fno.FnoError) as ei:
        fno.fno_spectral_conv2d_noalloc(x, w, 8, 8)
    assert ei.value.status == -2
