"""Seeded random shapes across the whole entry-point surface, each checked
against the fp64 oracle at the operator's bar (relative L2 <= 1e-5,
max-abs <= 1e-4 * max|ref|): sizes drawn from the power-of-two and
7-smooth lengths, ragged batch and channel counts, random mode counts
(including full modes), both transform orders of the layer tail."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import fft_spectral_convolution_amd as fno  # noqa: E402
import parity_log  # noqa: E402
from fft_spectral_convolution_amd.inputs import Config, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

REL_L2 = 1e-5
MAX_ABS = 1e-4
DEV = "cuda:0"
LENGTHS = [8, 12, 16, 20, 24, 30, 32, 36, 45, 48, 60, 64, 72, 96, 100, 128, 140, 256, 512]


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fno.lib()


def close(gpu, ref, what):
    g = gpu.detach().cpu().numpy()
    g = g.astype(np.complex128) if np.iscomplexobj(g) else g.astype(np.float64)
    rel = np.linalg.norm((g - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    mx = np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300)
    print(f"  {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    parity_log.record(what, rel, mx)
    assert rel <= REL_L2 and mx <= MAX_ABS, what


def draw_2d(rng):
    h, w = int(rng.choice(LENGTHS)), int(rng.choice(LENGTHS))
    if h * w > 128 * 256:
        h = min(h, 64)
    mx = int(rng.integers(1, h // 2 + 1))
    my = int(rng.integers(1, w // 2 + 2))
    b, cin, cout = int(rng.integers(1, 6)), int(rng.integers(1, 9)), int(rng.integers(1, 9))
    if rng.random() < 0.3:                      # the matrix-core mix
        b, cin, cout = int(rng.integers(8, 20)), int(rng.integers(8, 40)), 2 * int(rng.integers(8, 20))
    return Config("rand", "2d", b, cin, cout, h, w, mx, my, "uniform")


@pytest.mark.parametrize("seed", range(30))
def test_random_operator_and_backward_2d(seed):
    rng = np.random.default_rng(1000 + seed)
    cfg = draw_2d(rng)
    print(f"\n[{seed}] {cfg.describe()}", flush=True)
    x, w = make_inputs(cfg, seed)
    xd, wd = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (x, w))
    out = fno.fno_spectral_conv2d(xd, wd, cfg.mx, cfg.my)
    torch.cuda.synchronize()
    close(out, oracle.spectral_conv2d_ref(x, w, cfg.mx, cfg.my), "forward")
    g = rng.uniform(-1, 1, size=cfg.out_shape).astype(np.float32)
    gx, gw = fno.fno_spectral_conv2d_backward(xd, wd, torch.from_numpy(g).to(DEV), cfg.mx, cfg.my)
    torch.cuda.synchronize()
    rx, rw = oracle.spectral_conv2d_backward_ref(x, w, g, cfg.mx, cfg.my)
    close(gx, rx, "grad_x")
    close(gw, rw, "grad_w")


@pytest.mark.parametrize("seed", range(20))
def test_random_layer_and_filter_2d(seed):
    rng = np.random.default_rng(2000 + seed)
    cfg = draw_2d(rng)
    cfg = Config("rand", "2d", cfg.B, cfg.Cin, cfg.Cin, cfg.H, cfg.W, cfg.mx, cfg.my, "uniform")
    print(f"\n[{seed}] {cfg.describe()}", flush=True)
    x, w = make_inputs(cfg, seed)
    xd, wd = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (x, w))
    bias = rng.standard_normal(cfg.Cout).astype(np.float32)
    branch = rng.standard_normal(cfg.out_shape).astype(np.float32)
    after = bool(seed % 2)
    out = fno.fno_spectral_conv2d_gelu(xd, wd, cfg.mx, cfg.my, bias=torch.from_numpy(bias).to(DEV),
                                       branch=torch.from_numpy(branch).to(DEV), branch_after=after)
    torch.cuda.synchronize()
    close(out, oracle.spectral_conv2d_gelu_ref(x, w, cfg.mx, cfg.my, bias=bias, branch=branch, branch_after=after),
          "layer tail")
    mask = (rng.standard_normal((2, cfg.mx, cfg.my, cfg.Cin)) + 1j * rng.standard_normal((2, cfg.mx, cfg.my, cfg.Cin))
            ).astype(np.complex64)
    out = fno.fno_spectral_filter2d(xd, torch.from_numpy(mask).to(DEV), cfg.mx, cfg.my)
    torch.cuda.synchronize()
    close(out, oracle.spectral_filter2d_ref(x, mask, cfg.mx, cfg.my), "filter")


@pytest.mark.parametrize("seed", range(20))
def test_random_1d(seed):
    rng = np.random.default_rng(3000 + seed)
    n = int(rng.choice([8, 15, 16, 60, 64, 100, 128, 210, 256, 512, 1000, 1024, 2048, 2187, 4096]))
    modes = int(rng.integers(1, n // 2 + 2))
    b, cin, cout = int(rng.integers(1, 12)), int(rng.integers(1, 9)), int(rng.integers(1, 9))
    cfg = Config("rand1d", "1d", b, cin, cout, 1, n, 1, modes, "normal")
    print(f"\n[{seed}] {cfg.describe()}", flush=True)
    x, w = make_inputs(cfg, seed)
    xd, wd = (torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in (x, w))
    out = fno.fno_spectral_conv1d(xd, wd, modes)
    torch.cuda.synchronize()
    close(out, oracle.spectral_conv1d_ref(x, w, modes), "forward 1d")
    g = rng.standard_normal(cfg.out_shape).astype(np.float32)
    gx, gw = fno.fno_spectral_conv1d_backward(xd, wd, torch.from_numpy(g).to(DEV), modes)
    torch.cuda.synchronize()
    rx, rw = oracle.spectral_conv1d_backward_ref(x, w, g, modes)
    close(gx, rx, "grad_x 1d")
    close(gw, rw, "grad_w 1d")


@pytest.mark.parametrize("seed", range(15))
def test_random_linear_conv(seed):
    rng = np.random.default_rng(4000 + seed)
    h, w = int(rng.integers(1, 90)), int(rng.integers(1, 90))
    kh, kw = int(rng.integers(1, 10)), int(rng.integers(1, 10))
    b, cin, cout = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 6))
    x = rng.uniform(-1, 1, (b, cin, h, w)).astype(np.float32)
    k = rng.standard_normal((cout, cin, kh, kw)).astype(np.float32)
    fh, fw = h + kh - 1, w + kw - 1
    ch, cw = int(rng.integers(0, fh)), int(rng.integers(0, fw))
    ho, wo = int(rng.integers(1, fh - ch + 1)), int(rng.integers(1, fw - cw + 1))
    print(f"\n[{seed}] {b}x{cin}x{h}x{w} * {cout}x{cin}x{kh}x{kw}, window ({ch},{cw}) {ho}x{wo}", flush=True)
    out = fno.fno_linear_conv2d(torch.from_numpy(x).to(DEV), torch.from_numpy(k).to(DEV), crop=(ch, cw),
                                out_size=(ho, wo))
    torch.cuda.synchronize()
    close(out, oracle.linear_conv2d_ref(x, k, ch, cw, ho, wo), "linear conv")
