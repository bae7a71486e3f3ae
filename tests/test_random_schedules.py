"""Seeded random shapes drawn per schedule class, against the oracle.

The fixed edge cases in test_parity.py pin the boundaries each kernel was
written for, and test_random_shapes.py draws from the lengths of the whole
entry-point surface; this sweep draws from the shape space each specialised
schedule accepts (the one-kernel small call, the three-kernel small grids,
the pruned tall-grid columns and the pruned long rows: grid sides, kept
modes, channel and batch counts), so that an index that is right only at the
chosen edges shows up.  Shapes are drawn
from a fixed seed: every run checks the same cases.  Bar as in
test_parity.py (rel-L2 <= 1e-5, max-abs <= 1e-4 max|ref|).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import fft_spectral_convolution_amd as fno  # noqa: E402
import parity_log  # noqa: E402
from fft_spectral_convolution_amd.inputs import Config, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_L2 = 1e-5
MAX_ABS = 1e-4


def _draw_2d(rng, kind):
    """One 2D shape of a schedule class:
    'one'   grids of <= 1024 points, <= 8 channels (the one-kernel call),
    'small' grids up to 128 per side (three kernels),
    'tall'  2048..512-row grids whose kept kx suit the pruned columns,
    'wide'  512..4096-point rows (pruned long rows)."""
    if kind == "one":
        lh = int(rng.integers(3, 8))
        lw = int(rng.integers(3, 11 - lh)) if lh < 8 else 3
        lw = min(lw, 7)
        cin, cout = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        b = int(rng.integers(1, 6))
    elif kind == "small":
        lh, lw = int(rng.integers(5, 8)), int(rng.integers(5, 8))
        cin, cout = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        b = int(rng.integers(1, 5))
    elif kind == "tall":
        lh, lw = int(rng.integers(9, 12)), int(rng.integers(3, 6))
        cin, cout = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        b = 1
    else:
        lh, lw = int(rng.integers(1, 4)), int(rng.integers(9, 13))
        cin, cout = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        b = 1
    h, w = 1 << lh, 1 << lw
    if kind == "tall":
        q = h // 64                                  # 2 mx a multiple of the rows per lane
        mx = int(q // 2 * rng.integers(1, max(2, 128 // q)))
        mx = max(1, min(mx, 64, h // 2))
    else:
        mx = int(rng.integers(1, h // 2 + 1))
    my_max = w // 2 + 1
    if kind in ("tall", "wide"):
        my_max = min(my_max, 64)
    my = int(rng.integers(1, my_max + 1))
    return (b, cin, cout, h, w, mx, my)


def _cases_2d():
    rng = np.random.default_rng(20261203)
    out = []
    for kind, n in (("one", 14), ("small", 6), ("tall", 5), ("wide", 5)):
        for _ in range(n):
            out.append((kind,) + _draw_2d(rng, kind))
    return out


def _cases_1d():
    rng = np.random.default_rng(1203)
    out = []
    for _ in range(10):
        n = 1 << int(rng.integers(9, 13))            # the pruned long-row lengths
        modes = int(rng.integers(1, 65))
        out.append((int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(1, 9)), n, modes))
    for _ in range(4):
        n = 1 << int(rng.integers(3, 9))             # short rows (generic staged kernels)
        modes = int(rng.integers(1, n // 2 + 2))
        out.append((int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(1, 9)), n, modes))
    return out


def _check(got, ref, what):
    g = got.detach().cpu().numpy().astype(np.float64)
    rel = np.linalg.norm((g - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    mx = np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300)
    print(f"  {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    parity_log.record(what, rel, mx)
    assert rel <= REL_L2 and mx <= MAX_ABS, f"{what}: rel {rel:.3e}, max {mx:.3e}"


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fno.lib()


@pytest.mark.parametrize("case", _cases_2d(), ids=lambda c: c[0] + "-" + "x".join(map(str, c[1:])))
def test_random_shape_2d(case):
    kind, b, cin, cout, h, w, mx, my = case
    cfg = Config("rand2d", "2d", b, cin, cout, h, w, mx, my, "uniform")
    x, wt = make_inputs(cfg, 5)
    got = fno.fno_spectral_conv2d(torch.from_numpy(x).to(DEV), torch.from_numpy(wt).to(DEV), mx, my)
    torch.cuda.synchronize()
    _check(got, oracle.spectral_conv2d_ref(x, wt, mx, my), f"random 2d {kind} {case[1:]}")


@pytest.mark.parametrize("case", _cases_1d(), ids=lambda c: "x".join(map(str, c)))
def test_random_shape_1d(case):
    b, cin, cout, n, modes = case
    cfg = Config("rand1d", "1d", b, cin, cout, 1, n, 1, modes, "normal")
    x, wt = make_inputs(cfg, 6)
    got = fno.fno_spectral_conv1d(torch.from_numpy(x).to(DEV), torch.from_numpy(wt).to(DEV), modes)
    torch.cuda.synchronize()
    _check(got, oracle.spectral_conv1d_ref(x, wt, modes), f"random 1d {case}")
