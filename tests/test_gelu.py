"""GPU parity of the fused layer tail (fno_spectral_conv2d_gelu / _1d_gelu:
GELU of the spectral convolution plus bias, with a second branch added
before or after the activation) against the fp64 oracle, which the CPU suite
pins by normal-CDF table values and a DC-identity closed form.  Same bar as
the plain operator: relative L2 error <= 1e-5 and max-abs error <=
1e-4 * max|ref|.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import fft_spectral_convolution_amd as fno  # noqa: E402
import parity_log  # noqa: E402
from fft_spectral_convolution_amd.inputs import CONFIGS, Config, make_inputs  # noqa: E402

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
    g = gpu.detach().cpu().numpy().astype(np.float64)
    rel = np.linalg.norm((g - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    mx = np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300)
    print(f"  {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    parity_log.record(what, rel, mx)
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max-abs error {mx:.3e} > {MAX_ABS} * max|ref|"


def check(cfg, seed=0, use_bias=True, use_branch=True, branch_after=False):
    x, w = make_inputs(cfg, seed)
    rng = np.random.default_rng(seed + 200)
    out_shape = (cfg.B, cfg.Cout, cfg.W) if cfg.kind == "1d" else (cfg.B, cfg.Cout, cfg.H, cfg.W)
    bias = rng.standard_normal(cfg.Cout).astype(np.float32) if use_bias else None
    branch = rng.standard_normal(out_shape).astype(np.float32) if use_branch else None
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    xd, wd, bd, rd = dev(x), dev(w), dev(bias), dev(branch)
    if cfg.kind == "1d":
        out = fno.fno_spectral_conv1d_gelu(xd, wd, cfg.my, bias=bd, branch=rd, branch_after=branch_after)
        ref = oracle.spectral_conv1d_gelu_ref(x, w, cfg.my, bias=bias, branch=branch, branch_after=branch_after)
    else:
        out = fno.fno_spectral_conv2d_gelu(xd, wd, cfg.mx, cfg.my, bias=bd, branch=rd, branch_after=branch_after)
        ref = oracle.spectral_conv2d_gelu_ref(x, w, cfg.mx, cfg.my, bias=bias, branch=branch,
                                              branch_after=branch_after)
    torch.cuda.synchronize()
    assert fno.fno_last_kernels()[-1].endswith("_gelu")
    assert_close(out, ref, f"{cfg.name} gelu(branch_after={branch_after})")


@pytest.mark.parametrize("branch_after", [False, True])
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_gelu_workloads(name, branch_after):
    cfg = CONFIGS[name]
    print(f"\n[{name} gelu] {cfg.describe()}", flush=True)
    check(cfg, branch_after=branch_after)


GELU_2D = [
    # B, Cin, Cout, H, W, mx, my      (inverse kernel that applies the tail)
    (2, 3, 5, 8, 8, 4, 5),            # small-grid kernel, Nyquist column kept
    (3, 4, 6, 32, 16, 3, 9),          # small-grid kernel
    (2, 8, 16, 64, 64, 16, 16),       # one row per thread
    (2, 4, 6, 64, 128, 8, 20),        # one row per thread, 64 x 128
    (1, 2, 3, 256, 256, 9, 11),       # staged: 256-point short rows, generic columns (odd mx)
    (1, 2, 3, 128, 256, 9, 100),      # staged: generic rows (more than 64 bins)
    (1, 2, 3, 256, 64, 8, 12),        # staged: 64-point short rows, 256-row pruned columns
    (16, 8, 8, 256, 256, 8, 12),      # one-kernel 256 x 256 transforms (128 images), the tail in the inverse
    (16, 8, 8, 256, 256, 8, 24),      # one-kernel 256 x 256 transforms, two column blocks, the tail
    (16, 8, 8, 256, 512, 16, 24),     # one-kernel 256 x 512 transforms, two column blocks, the tail
    (16, 8, 8, 256, 512, 8, 12),      # one-kernel 256 x 512 transforms, one column block, the tail
    (16, 8, 8, 512, 512, 8, 16),      # one-kernel 512 x 512 transforms, the tail
    (16, 8, 8, 512, 256, 8, 12),      # one-kernel 512 x 256 transforms, the tail
    (16, 8, 8, 128, 256, 8, 24),      # one-kernel 128 x 256 transforms, the tail
    (16, 8, 8, 256, 128, 16, 20),     # one-kernel 256 x 128 transforms, the tail
    (16, 8, 8, 512, 128, 8, 12),      # one-kernel 512 x 128 transforms, the tail
    (1, 2, 3, 16, 1024, 5, 50),       # staged: pruned long rows
    (1, 2, 2, 1024, 16, 8, 9),        # staged: pruned columns, generic rows
    (2, 3, 4, 45, 100, 10, 20),       # mixed-radix rows and columns
]


@pytest.mark.parametrize("shape", GELU_2D, ids=lambda s: "x".join(map(str, s)))
def test_gelu_shapes_2d(shape):
    b, cin, cout, h, w, mx, my = shape
    check(Config("gelu", "2d", b, cin, cout, h, w, mx, my, "uniform"), 7, branch_after=bool(h % 3))


GELU_1D = [
    # B, Cin, Cout, N, modes
    (3, 2, 5, 16, 9),                 # generic rows, every bin kept
    (5, 3, 2, 512, 64),               # 512-point short rows
    (3, 2, 3, 256, 64),               # 256-point short rows, ragged last group of four rows
    (3, 2, 3, 512, 40),               # 512-point short rows, ragged last pair of rows
    (2, 3, 2, 256, 32),               # 256-point short rows, bins in the first two groups of 16
    (2, 2, 3, 512, 16),               # 512-point short rows, bins in the first group of 16 only
    (2, 2, 2, 512, 20),               # 512-point short rows, bins in the first two groups of 16
    (3, 2, 3, 64, 20),                # 64-point short rows, ragged last group of 16 rows
    (3, 2, 3, 128, 40),               # 128-point short rows, ragged last group of 8 rows
    (2, 4, 3, 4096, 33),              # pruned rows, longest
]


@pytest.mark.parametrize("shape", GELU_1D, ids=lambda s: "x".join(map(str, s)))
def test_gelu_shapes_1d(shape):
    b, cin, cout, n, modes = shape
    check(Config("gelu1d", "1d", b, cin, cout, 1, n, 1, modes, "normal"), 8, branch_after=bool(n % 3))


@pytest.mark.parametrize("use_bias,use_branch", [(False, False), (True, False), (False, True)])
def test_gelu_optional_terms(use_bias, use_branch):
    check(Config("gelu", "2d", 2, 8, 16, 128, 128, 8, 8, "uniform"), 9, use_bias=use_bias, use_branch=use_branch)
    check(Config("gelu1d", "1d", 4, 3, 4, 1, 2048, 1, 20, "normal"), 10, use_bias=use_bias, use_branch=use_branch)


@pytest.mark.parametrize("kind,shape", [
    ("2d", (1, 1, 2, 64, 64, 8, 8)),        # one row per thread
    ("2d", (1, 1, 2, 32, 32, 4, 4)),        # small-grid kernel
    ("2d", (1, 1, 2, 256, 256, 4, 4)),      # staged, 256-point short rows and pruned columns
    ("1d", (1, 1, 2, 1, 2048, 1, 16)),      # pruned long rows
])
def test_gelu_activation_accuracy(kind, shape):
    # x = 0 makes the transform chain exactly zero, so out = gelu(branch):
    # the device activation against the exact erf form over [-12, 12]
    b, cin, cout, h, w, mx, my = shape
    out_shape = (b, cout, w) if kind == "1d" else (b, cout, h, w)
    n = int(np.prod(out_shape))
    u = np.linspace(-12.0, 12.0, n).astype(np.float32).reshape(out_shape)
    xd = torch.zeros((b, cin, w) if kind == "1d" else (b, cin, h, w), device=DEV)
    if kind == "1d":
        wd = torch.ones((my, cin, cout), dtype=torch.complex64, device=DEV)
        out = fno.fno_spectral_conv1d_gelu(xd, wd, my, branch=torch.from_numpy(u).to(DEV))
    else:
        wd = torch.ones((2, mx, my, cin, cout), dtype=torch.complex64, device=DEV)
        out = fno.fno_spectral_conv2d_gelu(xd, wd, mx, my, branch=torch.from_numpy(u).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.gelu(u.astype(np.float64))
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    bound = 1e-6 * np.maximum(1.0, np.abs(u.astype(np.float64)))
    worst = int(np.argmax(err / bound))
    print(f"  max err {err.max():.3e}; worst ratio {float((err / bound).ravel()[worst]):.3f} at u={u.ravel()[worst]:.4f}")
    assert np.all(err <= bound)
