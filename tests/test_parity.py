"""GPU parity: libfno (through its C ABI) against the fp64 oracle.

Bar (fp32 path): relative L2 error <= 1e-5 and max-abs error <= 1e-4 * max|ref|,
on the same seeded fp32 / complex64 inputs.  Every workload shape runs at its
full size in the launch configuration the benchmark times; stage calls are
compared spectrum by spectrum (FFT blog, section 6.4: dump the intermediate
spectra and compare them point by point).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import fft_spectral_convolution_amd as fno  # noqa: E402
import parity_log  # noqa: E402
from fft_spectral_convolution_amd.inputs import CONFIGS, Config, make_inputs, make_weight, make_x  # noqa: E402

pytestmark = pytest.mark.gpu

REL_L2 = 1e-5
MAX_ABS = 1e-4

DEV = "cuda:0"


def errors(gpu, ref):
    g = gpu.detach().cpu().numpy()
    g = g.astype(np.complex128) if np.iscomplexobj(g) else g.astype(np.float64)
    ref = np.asarray(ref)
    rel = np.linalg.norm((g - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300)
    mx = np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300)
    return rel, mx


def assert_close(gpu, ref, what):
    rel, mx = errors(gpu, ref)
    print(f"  {what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}", flush=True)
    parity_log.record(what, rel, mx)
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max-abs error {mx:.3e} > {MAX_ABS} * max|ref|"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run(cfg, x, w, variant):
    xd, wd = to_dev(x), to_dev(w)
    if cfg.kind == "1d":
        fn = fno.fno_spectral_conv1d if variant == "fused" else fno.fno_spectral_conv1d_unfused
        out = fn(xd, wd, cfg.my)
    else:
        fn = fno.fno_spectral_conv2d if variant == "fused" else fno.fno_spectral_conv2d_unfused
        out = fn(xd, wd, cfg.mx, cfg.my)
    torch.cuda.synchronize()
    return out


def ref_out(cfg, x, w):
    if cfg.kind == "1d":
        return oracle.spectral_conv1d_ref(x, w, cfg.my)
    return oracle.spectral_conv2d_ref(x, w, cfg.mx, cfg.my)


_REF_CACHE = {}


def config_case(name):
    if name not in _REF_CACHE:
        cfg = CONFIGS[name]
        x, w = make_inputs(cfg, 0)
        _REF_CACHE.clear()
        _REF_CACHE[name] = (cfg, x, w, ref_out(cfg, x, w))
    return _REF_CACHE[name]


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fno.lib()


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_workload_parity(name, variant):
    cfg, x, w, ref = config_case(name)
    print(f"\n[{name} {variant}] {cfg.describe()}", flush=True)
    out = run(cfg, x, w, variant)
    assert_close(out, ref, f"{name} {variant} out")


# ---------------------------------------------------------------------------
# stage by stage
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c5"])
def test_stages_2d(name):
    cfg = CONFIGS[name]
    x, w = make_inputs(cfg, 0)
    xh_ref = oracle.forward_truncated_2d(x, cfg.mx, cfg.my)
    xh = fno.fno_forward2d(to_dev(x), cfg.mx, cfg.my)
    torch.cuda.synchronize()
    assert_close(xh, xh_ref, f"{name} forward spectrum")
    # each later stage starts from the same complex64 input on both sides
    xh32 = xh_ref.astype(np.complex64)
    yh_ref = oracle.mix_2d(xh32, w)
    yh = fno.fno_mix(to_dev(xh32), to_dev(w))
    torch.cuda.synchronize()
    assert_close(yh, yh_ref, f"{name} mixed spectrum")
    yh32 = yh_ref.astype(np.complex64)
    out_ref = oracle.inverse_from_truncated_2d(yh32, cfg.H, cfg.W)
    out = fno.fno_inverse2d(to_dev(yh32), cfg.H, cfg.W)
    torch.cuda.synchronize()
    assert_close(out, out_ref, f"{name} inverse")


@pytest.mark.parametrize("shape", [
    (16, 8, 8, 256, 256, 16, 32),   # the one-kernel 256 x 256 forward and inverse (128 images), two column blocks
    (16, 8, 8, 256, 512, 8, 12),    # the one-kernel 256 x 512 forward and inverse, one column block
    (16, 8, 8, 512, 512, 8, 16),    # the one-kernel 512 x 512 forward and inverse
    (16, 8, 8, 256, 128, 24, 16),   # the one-kernel 256 x 128 forward and inverse, one column block
    (16, 8, 8, 512, 128, 8, 16),    # the one-kernel 512 x 128 forward and inverse
    (2, 3, 4, 256, 256, 16, 32),    # few images: the staged transforms
], ids=lambda s: "x".join(map(str, s)))
def test_stages_2d_shapes(shape):
    b, cin, cout, h, wd, mx, my = shape
    cfg = Config("stage", "2d", b, cin, cout, h, wd, mx, my, "uniform")
    x, w = make_inputs(cfg, 3)
    xh = fno.fno_forward2d(to_dev(x), mx, my)
    torch.cuda.synchronize()
    assert_close(xh, oracle.forward_truncated_2d(x, mx, my), f"{shape} forward spectrum")
    yh32 = oracle.mix_2d(oracle.forward_truncated_2d(x, mx, my).astype(np.complex64), w).astype(np.complex64)
    out = fno.fno_inverse2d(to_dev(yh32), h, wd)
    torch.cuda.synchronize()
    assert_close(out, oracle.inverse_from_truncated_2d(yh32, h, wd), f"{shape} inverse")


@pytest.mark.parametrize("name", ["s1d", "c4"])
def test_stages_1d(name):
    # s1d: a 1024-point sequence with a ragged mode count; c4: the full
    # token-mixing workload (4096 points, 64 modes, 256 x 64 rows)
    if name == "c4":
        cfg = CONFIGS["c4"]
        x, w = make_inputs(cfg, 0)
    else:
        cfg = Config("s1d", "1d", 8, 16, 12, 1, 1024, 1, 40, "normal")
        x, w = make_inputs(cfg, 3)
    xh_ref = oracle.forward_truncated_1d(x, cfg.my)
    xh = fno.fno_forward1d(to_dev(x), cfg.my)
    torch.cuda.synchronize()
    assert_close(xh, xh_ref, f"{name} forward spectrum")
    xh32 = xh_ref.astype(np.complex64)
    yh_ref = oracle.mix_1d(xh32, w)
    yh = fno.fno_mix(to_dev(xh32), to_dev(w))
    torch.cuda.synchronize()
    assert_close(yh, yh_ref, f"{name} mixed spectrum")
    yh32 = yh_ref.astype(np.complex64)
    out = fno.fno_inverse1d(to_dev(yh32), cfg.W)
    torch.cuda.synchronize()
    assert_close(out, oracle.inverse_from_truncated_1d(yh32, cfg.W), f"{name} inverse")


# ---------------------------------------------------------------------------
# edge shapes: tiny grids, full modes, ragged tails, non-square, longest rows
# ---------------------------------------------------------------------------

EDGE_2D = [
    # B, Cin, Cout, H, W, mx, my
    (300, 2, 3, 32, 32, 8, 8),      # one-kernel small path: more batch items than CUs
    (2, 4, 4, 256, 256, 32, 32),    # few images: staged 256-point short rows and 256-row short columns
    (16, 8, 8, 256, 256, 32, 32),   # one-kernel 256 x 256 transforms (128 images), two column blocks
    (16, 8, 8, 256, 256, 16, 12),   # one-kernel 256 x 256 transforms, one column block
    (2, 3, 5, 256, 512, 16, 17),    # few images: staged 512-point short rows, one column in the last block
    (16, 8, 8, 256, 512, 16, 17),   # one-kernel 256 x 512 transforms, one column in the last block
    (16, 8, 8, 256, 512, 16, 16),   # one-kernel 256 x 512 transforms, one column block
    (2, 3, 2, 512, 256, 64, 64),    # 256-point short rows, every bin up to 64; 512-row short columns, 128 kept kx
    (16, 8, 8, 256, 256, 64, 16),   # one-kernel 256 x 256 transforms: every kept kx of 128, one column block
    (16, 8, 8, 256, 512, 8, 32),    # one-kernel 256 x 512 transforms: two column blocks
    (8, 64, 4, 256, 256, 8, 8),     # one-kernel 256 x 256 forward: more images than workgroups
    (4, 4, 96, 256, 256, 8, 20),    # one-kernel 256 x 256 inverse: more images than workgroups, ragged last block
    (16, 8, 8, 512, 512, 16, 16),   # one-kernel 512 x 512 transforms (16 kept columns, two phase blocks per column)
    (16, 8, 8, 512, 256, 8, 12),    # one-kernel 512 x 256 transforms, ragged column block
    (16, 8, 8, 128, 256, 16, 20),   # one-kernel 128 x 256 transforms, ragged second column block
    (16, 8, 8, 128, 256, 32, 12),   # one-kernel 128 x 256 transforms, every kx kept (64 of 128 rows)
    (16, 8, 8, 128, 256, 40, 12),   # 128 x 256 with more than 64 kept kx: staged transforms
    (16, 8, 8, 256, 128, 16, 20),   # one-kernel 256 x 128 transforms, ragged second column block
    (16, 8, 8, 256, 128, 64, 8),    # one-kernel 256 x 128 transforms, every kept kx of 128, one column block
    (16, 8, 8, 256, 128, 8, 32),    # one-kernel 256 x 128 transforms, two whole column blocks
    (40, 8, 8, 256, 128, 16, 20),   # 256 x 128 with more images than CUs: staged transforms
    (16, 8, 8, 512, 128, 16, 12),   # one-kernel 512 x 128 transforms, ragged column block
    (16, 8, 8, 512, 128, 64, 16),   # one-kernel 512 x 128 transforms, 128 kept kx, a whole column block
    (8, 24, 16, 512, 128, 16, 12),  # 512 x 128: 192 images in (staged forward), 128 out (one-kernel inverse)
    (16, 8, 8, 256, 128, 8, 1),     # one-kernel 256 x 128 transforms, one kept column
    (16, 8, 8, 512, 128, 8, 1),     # one-kernel 512 x 128 transforms, one kept column
    (1, 2, 3, 128, 256, 9, 100),    # 256-point rows with more than 64 bins: generic rows and columns
    (1, 2, 3, 512, 128, 24, 5),     # 512-row short columns, one partial block of 16 columns
    (2, 3, 4, 256, 64, 8, 20),      # 64-point short rows (16 rows per wave), bins in two groups of 16
    (2, 3, 4, 512, 64, 16, 32),     # 64-point short rows, every bin below the Nyquist bin
    (1, 2, 3, 256, 64, 8, 33),      # 64-point rows keeping the Nyquist bin: generic rows
    (2, 2, 3, 256, 128, 16, 64),    # 128-point short rows, every bin up to 64
    (2, 3, 4, 128, 256, 16, 20),    # 128-row short columns (8 phases per thread), ragged column block
    (2, 3, 4, 64, 512, 8, 12),      # 64-row short columns (4 phases per thread)
    (1, 2, 3, 128, 512, 32, 64),    # 128-row short columns, four modes per residue
    (1, 2, 2, 128, 256, 64, 8),     # 128-row short columns, every kx kept
    (4, 160, 160, 256, 128, 8, 40), # 256-row short columns: more column blocks than workgroups, ragged last block
    (3, 100, 100, 512, 128, 8, 40), # 512-row short columns: more column blocks than workgroups
    (5, 8, 8, 32, 32, 16, 16),      # one-kernel small path: most channels (two rounds), every kx kept
    (4, 7, 1, 16, 64, 8, 17),       # one-kernel small path: one output channel (idle groups in the inverse)
    (2, 3, 3, 8, 128, 2, 40),       # one-kernel small path: 8 x 128 grid
    (3, 1, 8, 8, 32, 4, 17),        # one-kernel small path: one input channel, Nyquist column kept
    (1, 1, 1, 2, 2, 1, 1),
    (1, 1, 1, 2, 2, 1, 2),          # full modes of a 2x2 grid (Nyquist column kept)
    (3, 5, 7, 8, 8, 4, 5),          # full modes, odd channel counts
    (2, 3, 2, 16, 64, 3, 33),       # non-square, Nyquist column kept
    (2, 2, 3, 64, 8, 32, 2),        # tall grid, every kx kept
    (5, 3, 65, 32, 32, 5, 7),       # Cout beyond one 64-wide tile, ragged batch tile
    (1, 2, 2, 4096, 4, 3, 2),       # longest columns
    (1, 2, 1, 4, 4096, 2, 100),     # longest rows
    (9, 1, 1, 128, 128, 64, 65),    # odd batch, full modes
    (9, 12, 18, 16, 16, 3, 5),      # matrix-core mix: ragged batch, channels and modes (30 modes)
    (40, 16, 34, 32, 32, 4, 4),     # matrix-core mix: two batch tiles, ragged output tile
    (33, 64, 66, 64, 64, 8, 8),     # matrix-core mix: 64+2 output channels, 33 batch rows
    (3, 2, 5, 128, 128, 7, 13),     # one-row-per-thread forward: ragged column batch
    (2, 3, 4, 64, 64, 32, 32),      # one-row-per-thread forward: every kx kept, two column batches
    (2, 2, 2, 128, 64, 5, 17),      # one-row-per-thread forward: tall, my just past one batch
    (2, 2, 2, 64, 128, 9, 3),       # one-row-per-thread forward: wide rows, few columns
    (1, 2, 3, 16, 1024, 5, 50),     # pruned long rows (1024 points), ragged last bin chunk
    (1, 1, 2, 8, 4096, 2, 64),      # pruned long rows at the longest length, every chunk
    (1, 2, 3, 1024, 16, 8, 9),      # pruned columns (1024 rows), ragged column block
    (2, 2, 2, 512, 32, 4, 7),       # pruned columns (512 rows), few kept rows
    (1, 1, 2, 1024, 8, 5, 3),       # tall grid whose kept rows do not suit the pruned columns
    (1, 2, 2, 2048, 128, 64, 60),   # pruned columns at the large-grid row count, 128 kept rows
    (8, 64, 64, 128, 128, 32, 32),  # matrix-core mix: 16-row tiles of 64 output channels
    (64, 16, 32, 128, 128, 32, 32), # matrix-core mix: 32-row tiles of 32 output channels
]


@pytest.mark.parametrize("shape", EDGE_2D, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_edge_shapes_2d(shape, variant):
    b, cin, cout, h, wd, mx, my = shape
    cfg = Config("edge", "2d", b, cin, cout, h, wd, mx, my, "uniform")
    x, w = make_inputs(cfg, 7)
    out = run(cfg, x, w, variant)
    assert_close(out, ref_out(cfg, x, w), f"edge {shape} {variant}")


EDGE_1D = [
    # B, Cin, Cout, N, modes
    (1, 1, 1, 2, 1),
    (1, 1, 1, 2, 2),
    (3, 1, 2, 16, 9),               # odd number of rows, full modes
    (7, 3, 5, 64, 17),              # odd rows B*Cin = 21
    (2, 4, 70, 4096, 2049),         # longest sequence, every bin kept
    (33, 2, 3, 256, 1),             # DC only, short rows with a ragged last group of four
    (5, 3, 2, 512, 64),             # 512-point short rows, every bin up to 64, odd forward row count
    (3, 2, 3, 1024, 1),             # pruned rows, DC only
    (4, 3, 5, 2048, 37),            # pruned rows, partial last chunk of 16 bins
    (2, 2, 3, 2048, 16),            # pruned rows: only the first 16 residues staged
    (3, 2, 3, 256, 64),             # 256-point short rows, every bin up to 64
    (2, 3, 2, 256, 33),             # 256-point short rows, odd mode count
    (3, 2, 3, 512, 17),             # 512-point short rows, one bin past the first 16, odd row counts
    (2, 2, 3, 512, 16),             # 512-point short rows, bins in the first group of 16 only
    (7, 3, 5, 64, 32),              # 64-point short rows, ragged last group of 16 rows
    (4, 2, 3, 64, 33),              # 64-point rows keeping the Nyquist bin: generic rows
    (5, 3, 2, 128, 64),             # 128-point short rows, every bin up to 64
    (3, 2, 3, 128, 65),             # 128-point rows keeping the Nyquist bin: generic rows
    (9, 3, 1, 128, 7),              # 128-point short rows, one output channel, ragged groups of 8 rows
    (3, 1, 2, 1024, 17),            # pruned rows: one bin in the second group of each residue
    (9, 2, 2, 4096, 17),            # pruned rows, odd row count
]


@pytest.mark.parametrize("shape", EDGE_1D, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("variant", ["fused", "unfused"])
def test_edge_shapes_1d(shape, variant):
    b, cin, cout, n, modes = shape
    cfg = Config("edge1d", "1d", b, cin, cout, 1, n, 1, modes, "normal")
    x, w = make_inputs(cfg, 11)
    out = run(cfg, x, w, variant)
    assert_close(out, ref_out(cfg, x, w), f"edge1d {shape} {variant}")


# lengths with prime factors 3, 5, 7 (mixed-radix stage kernels)
MIXED_2D = [
    # B, Cin, Cout, H, W, mx, my
    (2, 3, 4, 96, 96, 12, 12),      # 2^5 3
    (2, 4, 4, 100, 100, 16, 16),    # 2^2 5^2
    (1, 2, 3, 45, 63, 10, 20),      # odd lengths: no Nyquist column
    (2, 2, 2, 7, 5, 3, 3),          # prime lengths, every mode kept
    (1, 1, 2, 2187, 10, 20, 6),     # 3^7-row columns
    (1, 2, 2, 48, 1000, 24, 501),   # every mode of a 2^3 5^3 row kept
    (16, 16, 32, 120, 120, 16, 16), # matrix-core mix between mixed-radix transforms
]


@pytest.mark.parametrize("shape", MIXED_2D, ids=lambda s: "x".join(map(str, s)))
def test_mixed_radix_shapes_2d(shape):
    b, cin, cout, h, wd, mx, my = shape
    cfg = Config("mixed", "2d", b, cin, cout, h, wd, mx, my, "uniform")
    x, w = make_inputs(cfg, 13)
    out = run(cfg, x, w, "fused")
    assert_close(out, ref_out(cfg, x, w), f"mixed {shape}")


MIXED_1D = [
    # B, Cin, Cout, N, modes
    (3, 2, 3, 1000, 64),            # 2^3 5^3
    (2, 2, 2, 3125, 100),           # 5^5
    (2, 2, 2, 2401, 50),            # 7^4
    (4, 3, 3, 15, 8),               # odd length, every bin kept
    (8, 16, 16, 3072, 64),          # 2^10 3, matrix-core mix
]


@pytest.mark.parametrize("shape", MIXED_1D, ids=lambda s: "x".join(map(str, s)))
def test_mixed_radix_shapes_1d(shape):
    b, cin, cout, n, modes = shape
    cfg = Config("mixed1d", "1d", b, cin, cout, 1, n, 1, modes, "normal")
    x, w = make_inputs(cfg, 14)
    out = run(cfg, x, w, "fused")
    assert_close(out, ref_out(cfg, x, w), f"mixed1d {shape}")


def test_identity_full_modes_reproduces_input():
    rng = np.random.default_rng(5)
    b, c, h, wd = 2, 3, 32, 16
    x = make_x(rng, (b, c, h, wd), "uniform")
    w = np.broadcast_to(np.eye(c, dtype=np.complex64), (2, h // 2, wd // 2 + 1, c, c)).copy()
    out = fno.fno_spectral_conv2d(to_dev(x), to_dev(w), h // 2, wd // 2 + 1)
    torch.cuda.synchronize()
    assert_close(out, x.astype(np.float64), "identity, full modes")


# ---------------------------------------------------------------------------
# API behaviour
# ---------------------------------------------------------------------------

def test_deterministic():
    cfg, x, w, _ = config_case("c2")
    a = run(cfg, x, w, "fused")
    b = run(cfg, x, w, "fused")
    assert torch.equal(a, b)


def test_workspace_variant_and_stream():
    cfg = CONFIGS["c2"]
    x, w = make_inputs(cfg, 0)
    xd, wd = to_dev(x), to_dev(w)
    need = fno.fno_workspace_size_2d(cfg.B, cfg.Cin, cfg.Cout, cfg.H, cfg.W, cfg.mx, cfg.my)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = fno.fno_spectral_conv2d_ws(xd, wd, cfg.mx, cfg.my, ws)
    s.synchronize()
    ref = fno.fno_spectral_conv2d(xd, wd, cfg.mx, cfg.my)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    if need > 0:
        small = torch.empty(need - 256 if need > 256 else 1, dtype=torch.uint8, device=DEV)
        with pytest.raises(fno.FnoError) as ei:
            fno.fno_spectral_conv2d_ws(xd, wd, cfg.mx, cfg.my, small)
        assert ei.value.status == -8


def test_concurrent_streams_internal_workspace():
    # calls on two streams overlap in time; each stream has its own internal
    # workspace, so the results equal those of calls made one after another
    cfg = CONFIGS["c3"]
    x, w = make_inputs(cfg, 0)
    xd, wd = to_dev(x), to_dev(w)
    x2 = torch.flip(xd, dims=[0]).contiguous()
    ref1 = fno.fno_spectral_conv2d(xd, wd, cfg.mx, cfg.my)
    ref2 = fno.fno_spectral_conv2d(x2, wd, cfg.mx, cfg.my)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs1, outs2 = [], []
    for _ in range(3):
        with torch.cuda.stream(s1):
            outs1.append(fno.fno_spectral_conv2d(xd, wd, cfg.mx, cfg.my))
        with torch.cuda.stream(s2):
            outs2.append(fno.fno_spectral_conv2d(x2, wd, cfg.mx, cfg.my))
    torch.cuda.synchronize()
    for a, b in zip(outs1, outs2):
        assert torch.equal(a, ref1) and torch.equal(b, ref2)


def test_out_is_overwritten():
    cfg, x, w, ref = config_case("c1")
    out = torch.full(cfg.out_shape, float("nan"), dtype=torch.float32, device=DEV)
    fno.fno_spectral_conv2d(to_dev(x), to_dev(w), cfg.mx, cfg.my, out=out)
    torch.cuda.synchronize()
    assert_close(out, ref, "c1 into a NaN-filled out")


def test_bad_arguments_raise():
    x = torch.zeros((1, 2, 8, 22), device=DEV)          # W has the prime factor 11
    w = torch.zeros((2, 2, 2, 2, 2), dtype=torch.complex64, device=DEV)
    with pytest.raises(fno.FnoError) as ei:
        fno.fno_spectral_conv2d(x, w, 2, 2)
    assert ei.value.status == -2
    x = torch.zeros((1, 2, 8, 8), device=DEV)
    w = torch.zeros((2, 5, 2, 2, 2), dtype=torch.complex64, device=DEV)
    with pytest.raises(fno.FnoError) as ei:
        fno.fno_spectral_conv2d(x, w, 5, 2)               # 2*mx > H
    assert ei.value.status == -3


SCHEDULES = {
    "c1": ["conv_fused"],                                   # the whole call in one kernel
    "c2": ["fwd2d", "mix_mfma", "inv2d"],
    "c3": ["fwd2d", "mix_mfma", "inv2d"],
    "c4": ["rows_fwd", "mix_mfma", "rows_inv"],
    "c5": ["rows_fwd", "cols_fwd", "mix_valu", "cols_inv", "rows_inv"],
}


@pytest.mark.parametrize("name", sorted(SCHEDULES))
def test_schedule_selection(name):
    # which kernels the plain call launches for each workload shape (the
    # parity of each schedule is checked above; this pins the dispatch)
    cfg = CONFIGS[name]
    g = torch.Generator(device=DEV).manual_seed(0)
    x = torch.rand(cfg.x_shape, device=DEV, generator=g)
    w = torch.randn(cfg.w_shape, dtype=torch.complex64, device=DEV, generator=g)
    if cfg.kind == "1d":
        fno.fno_spectral_conv1d(x, w, cfg.my)
    else:
        fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my)
    torch.cuda.synchronize()
    assert fno.fno_last_kernels() == SCHEDULES[name]
    if name == "c1":
        # the ablation and the fused layer tail keep their own schedules
        fno.fno_spectral_conv2d_unfused(x, w, cfg.mx, cfg.my)
        assert fno.fno_last_kernels() == ["rows_fwd", "cols_fwd", "mix_valu", "cols_inv", "rows_inv"]
        fno.fno_spectral_conv2d_gelu(x, w, cfg.mx, cfg.my)
        assert fno.fno_last_kernels() == ["fwd2d", "mix_valu", "inv2d_gelu"]
