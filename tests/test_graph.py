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
    Config("g32f", "2d", 3, 4, 4, 32, 32, 8, 8, "uniform"),           # the whole call in one kernel
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


# ---------------------------------------------------------------------------
# allocation is refused during capture; host threads sharing a stream
# ---------------------------------------------------------------------------

def _captured_status(s, call, also):
    """Run call() inside a capture on stream s (with one ordinary kernel,
    also(), captured beside it); return the FnoError status it raised, or 0."""
    g = torch.cuda.CUDAGraph()
    status = 0
    with torch.cuda.graph(g, stream=s):
        also()
        try:
            call()
        except fno.FnoError as err:
            status = err.status
    torch.cuda.synchronize()
    return status


def test_capture_refuses_workspace_growth():
    # a fresh stream has no workspace yet: the call would allocate one
    cfg = Config("cap", "2d", 2, 8, 8, 64, 64, 8, 8, "uniform")
    x, w = _inputs(cfg, 0)
    out = torch.empty((cfg.B, cfg.Cout, cfg.H, cfg.W), device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    st = _captured_status(s, lambda: fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my, out=out), lambda: out.add_(1.0))
    assert st == -9, f"expected FNO_ERR_CAPTURE, got {st}"
    # the same call eagerly on that stream, then captured: allowed
    with torch.cuda.stream(s):
        ref = fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my)
    s.synchronize()
    st = _captured_status(s, lambda: fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my, out=out), lambda: out.add_(1.0))
    assert st == 0
    assert torch.isfinite(ref).all()


def test_capture_refuses_new_mixed_radix_table():
    # the workspace of the stream is large enough, but a 7-smooth length used
    # for the first time in this process needs its twiddle table built
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    big = Config("cap1d", "1d", 2, 4, 4, 1, 4096, 1, 64, "normal")
    xb, wb = _inputs(big, 0)
    with torch.cuda.stream(s):
        fno.fno_spectral_conv1d(xb, wb, big.my)
    s.synchronize()
    n = 2 * 3 * 5 * 7 * 3          # 630: not used by any other test
    odd = Config("cap630", "1d", 2, 4, 4, 1, n, 1, 32, "normal")
    x, w = _inputs(odd, 0)
    out = torch.empty((odd.B, odd.Cout, n), device=DEV)
    st = _captured_status(s, lambda: fno.fno_spectral_conv1d(x, w, odd.my, out=out), lambda: out.add_(1.0))
    assert st == -9, f"expected FNO_ERR_CAPTURE, got {st}"
    with torch.cuda.stream(s):
        fno.fno_spectral_conv1d(x, w, odd.my, out=out)     # builds the table eagerly
    s.synchronize()
    st = _captured_status(s, lambda: fno.fno_spectral_conv1d(x, w, odd.my, out=out), lambda: out.add_(1.0))
    assert st == 0


def test_threads_sharing_a_stream_grow_its_workspace():
    # Two host threads call on the same (new) stream at once, one with a
    # shape that needs a larger internal workspace than the other's: the
    # growth must wait until the other call's kernels are enqueued and done
    # before it frees the old buffer.  Every result must equal the eager one.
    import threading
    small = Config("thr_s", "2d", 2, 8, 8, 64, 64, 8, 8, "uniform")
    large = Config("thr_l", "2d", 4, 32, 32, 128, 128, 32, 32, "uniform")
    xs, ws = _inputs(small, 1)
    xl, wl = _inputs(large, 2)
    ref_s = fno.fno_spectral_conv2d(xs, ws, small.mx, small.my)
    ref_l = fno.fno_spectral_conv2d(xl, wl, large.mx, large.my)
    torch.cuda.synchronize()
    for it in range(8):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        outs_s = [torch.empty_like(ref_s) for _ in range(4)]
        outs_l = [torch.empty_like(ref_l) for _ in range(4)]
        errs = []

        def worker(outs, x, w, cfg):
            try:
                with torch.cuda.stream(s):
                    for o in outs:
                        fno.fno_spectral_conv2d(x, w, cfg.mx, cfg.my, out=o)
            except Exception as e:  # noqa: BLE001
                errs.append(e)
        ta = threading.Thread(target=worker, args=(outs_s, xs, ws, small))
        tb = threading.Thread(target=worker, args=(outs_l, xl, wl, large))
        ta.start()
        tb.start()
        ta.join()
        tb.join()
        s.synchronize()
        assert not errs, errs
        for o in outs_s:
            assert torch.equal(o, ref_s), f"iteration {it}: small call differs"
        for o in outs_l:
            assert torch.equal(o, ref_l), f"iteration {it}: large call differs"
