"""HIP graph capture of libfno calls.

A call captured into a graph (torch.cuda.CUDAGraph over HIP graphs) must
recompute on every replay from whatever its input buffers hold then.  Each
case warms the call up on the capturing stream (the per-stream internal
workspace and the twiddle tables are allocated then, never during capture),
captures it, and replays it several times with new inputs copied in, eager
work and synchronisations between the replays; every replay must equal, bit
for bit, an eager call of the same entry point on the same inputs (the
kernels and their launch shapes are the same, and every reduction runs in a
fixed order).  The eager results themselves are checked against the oracle
by the parity tests.
"""
import pytest

torch = pytest.importorskip("torch")

import fft_spectral_convolution_amd as fno  # noqa: E402
from fft_spectral_convolution_amd.inputs import Config, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fno.lib()


def _inputs(cfg, seed):
    x, w = make_inputs(cfg, seed=seed)
    return torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV)


def _replay_matches_eager(cfg, capture, eager, extra=None):
    """capture(x, w, e) -> output tensors written by the captured call;
    eager(x, w, e) -> fresh outputs of the same call, on the current stream.
    e: extra device inputs (the loss gradient), refreshed like x."""
    x, w = _inputs(cfg, 0)
    e = extra(cfg, 0) if extra else None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture(x, w, e)                  # warm-up on the capturing stream
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = capture(x, w, e)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        xn, wn = _inputs(cfg, 100 + rep)
        x.copy_(xn)
        w.copy_(wn)
        if extra:
            e.copy_(extra(cfg, 100 + rep))
        for o in outs:
            o.fill_(float("nan"))         # a replay that skips a write shows up
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager(xn, wn, extra(cfg, 100 + rep) if extra else None)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"{cfg.name}: replay {rep} differs from the eager call"
        print(f"  {cfg.name}: replay {rep} equal to the eager call", flush=True)


FORWARD_2D = [
    Config("g64", "2d", 4, 16, 16, 64, 64, 16, 16, "uniform"),         # one-thread-per-row kernels
    Config("g128", "2d", 2, 64, 64, 128, 128, 32, 32, "uniform"),      # matrix-core mix
    Config("g512", "2d", 1, 4, 4, 512, 512, 32, 32, "uniform"),        # pruned rows and columns
    Config("g96", "2d", 2, 8, 8, 96, 96, 12, 12, "uniform"),           # mixed-radix stages
]


@pytest.mark.parametrize("cfg", FORWARD_2D, ids=lambda c: c.name)
def test_graph_forward_2d(cfg):
    out = torch.empty((cfg.B, cfg.Cout, cfg.H, cfg.W), device=DEV)
    _replay_matches_eager(
        cfg,
        lambda x, w, e: (fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my, out=out),),
        lambda x, w, e: (fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my),))


def test_graph_forward_2d_caller_workspace():
    cfg = Config("g128ws", "2d", 2, 32, 32, 128, 128, 32, 32, "uniform")
    out = torch.empty((cfg.B, cfg.Cout, cfg.H, cfg.W), device=DEV)
    ws = torch.empty(max(fno.fno_workspace_size_2d(cfg.B, cfg.Cin, cfg.Cout, cfg.H, cfg.W, cfg.mx, cfg.my), 1),
                     dtype=torch.uint8, device=DEV)
    _replay_matches_eager(
        cfg,
        lambda x, w, e: (fno.fno_spectral_conv2d_ws(x, w, cfg.mx, cfg.my, ws, out=out),),
        lambda x, w, e: (fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my),))


def test_graph_forward_1d():
    cfg = Config("g1d", "1d", 16, 32, 32, 1, 4096, 1, 64, "normal")
    out = torch.empty((cfg.B, cfg.Cout, cfg.W), device=DEV)
    _replay_matches_eager(
        cfg,
        lambda x, w, e: (fno.fno_spectral_conv1d(x, w, cfg.my, out=out),),
        lambda x, w, e: (fno.fno_spectral_conv1d(x, w, cfg.my),))


def _grad_out(cfg, seed):
    g = torch.Generator().manual_seed(seed)
    shape = (cfg.B, cfg.Cout, cfg.W) if cfg.kind == "1d" else (cfg.B, cfg.Cout, cfg.H, cfg.W)
    return torch.randn(shape, generator=g).to(DEV)


@pytest.mark.parametrize("cfg", [
    Config("gb128", "2d", 2, 64, 64, 128, 128, 32, 32, "uniform"),
    Config("gb1d", "1d", 8, 32, 32, 1, 2048, 1, 64, "normal"),
], ids=lambda c: c.name)
def test_graph_backward(cfg):
    gx = torch.empty((cfg.B, cfg.Cin, cfg.W) if cfg.kind == "1d" else (cfg.B, cfg.Cin, cfg.H, cfg.W), device=DEV)
    gw = torch.empty(cfg.w_shape, dtype=torch.complex64, device=DEV)
    if cfg.kind == "1d":
        cap = lambda x, w, e: fno.fno_spectral_conv1d_backward(x, w, e, cfg.my, grad_x=gx, grad_w=gw)  # noqa: E731
        eag = lambda x, w, e: fno.fno_spectral_conv1d_backward(x, w, e, cfg.my)  # noqa: E731
    else:
        cap = lambda x, w, e: fno.fno_spectral_conv2d_backward(x, w, e, cfg.mx, cfg.my, grad_x=gx, grad_w=gw)  # noqa: E731
        eag = lambda x, w, e: fno.fno_spectral_conv2d_backward(x, w, e, cfg.mx, cfg.my)  # noqa: E731
    _replay_matches_eager(cfg, cap, eag, extra=_grad_out)
