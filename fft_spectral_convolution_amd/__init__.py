"""Python binding of libfno, the MI355X (gfx950) spectral-convolution library.

Thin ctypes marshalling over the C ABI declared in include/fno.h: the
functions here have the ABI's names, take torch tensors for device memory
and the current torch stream, and do no arithmetic themselves.  Every step of
the operator runs in the library's HIP kernels.  If libfno.so is missing or
cannot be loaded, every call raises; there is no fallback.

    import fft_spectral_convolution_amd as fno
    out = fno.fno_spectral_conv2d(x, w, mx, my)      # x [B,Cin,H,W] f32, w [2,mx,my,Cin,Cout] c64
    out = fno.fno_spectral_conv1d(x, w, modes)       # x [B,Cin,N]   f32, w [modes,Cin,Cout]   c64
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

__all__ = [
    "FnoError",
    "lib",
    "library_path",
    "fno_version",
    "fno_status_string",
    "fno_init",
    "fno_spectral_conv2d",
    "fno_spectral_conv1d",
    "fno_spectral_conv2d_unfused",
    "fno_spectral_conv1d_unfused",
    "fno_spectral_conv2d_ws",
    "fno_spectral_conv2d_noalloc",
    "fno_noalloc_scratch_bytes",
    "fno_spectral_conv1d_ws",
    "fno_spectral_conv2d_backward",
    "fno_spectral_conv1d_backward",
    "fno_spectral_conv2d_gelu",
    "fno_spectral_conv1d_gelu",
    "fno_spectral_filter2d",
    "fno_spectral_filter1d",
    "fno_linear_conv_length",
    "fno_linear_conv2d_prepare",
    "fno_linear_conv2d",
    "fno_linear_conv1d_prepare",
    "fno_linear_conv1d",
    "fno_workspace_size_2d",
    "fno_workspace_size_1d",
    "fno_forward2d",
    "fno_inverse2d",
    "fno_forward1d",
    "fno_inverse1d",
    "fno_mix",
    "fno_set_timing_events",
    "fno_last_kernels",
    "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfno.so"

_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_S = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/fno.h
_SIGNATURES = {
    "fno_version": (_I, []),
    "fno_status_string": (ctypes.c_char_p, [_I]),
    "fno_last_hip_error": (_I, []),
    "fno_init": (_I, []),
    "fno_spectral_conv2d": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_conv1d": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_conv2d_unfused": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_conv1d_unfused": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fno_workspace_size_2d": (_S, [_I, _I, _I, _I, _I, _I, _I]),
    "fno_workspace_size_1d": (_S, [_I, _I, _I, _I, _I]),
    "fno_spectral_conv2d_ws": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _S, _P]),
    "fno_spectral_conv2d_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fno_noalloc_scratch_bytes": (_S, []),
    "fno_spectral_conv1d_ws": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _S, _P]),
    "fno_forward2d": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fno_mix": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "fno_inverse2d": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fno_forward1d": (_I, [_P, _P, _I, _I, _I, _I, _P]),
    "fno_inverse1d": (_I, [_P, _P, _I, _I, _I, _I, _P]),
    "fno_spectral_conv2d_backward": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_conv1d_backward": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_conv2d_gelu": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_conv1d_gelu": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_filter2d": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fno_spectral_filter1d": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "fno_linear_conv_length": (_I, [_I, _I]),
    "fno_linear_conv2d_prepare": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fno_linear_conv2d": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fno_linear_conv1d_prepare": (_I, [_P, _P, _I, _I, _I, _I, _P]),
    "fno_linear_conv1d": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fno_set_timing_events": (_I, [ctypes.POINTER(ctypes.c_void_p), _I]),
    "fno_last_kernel_count": (_I, []),
    "fno_last_kernel_name": (ctypes.c_char_p, [_I]),
}

EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class FnoError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: libfno status {status}: {message}")
        self.status = status


def library_path() -> str:
    return os.environ.get("LIBFNO_PATH", os.path.join(_HERE, _LIB_NAME))


def lib() -> ctypes.CDLL:
    """The loaded libfno.so (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise ImportError(
                    f"{path} is missing: build the HIP library first "
                    "(python -m fft_spectral_convolution_amd.build)")
            handle = ctypes.CDLL(path)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def fno_version() -> int:
    return lib().fno_version()


def fno_status_string(status: int) -> str:
    return lib().fno_status_string(status).decode()


def fno_init() -> None:
    """Build the current device's twiddle table now (a later call may then be
    captured into a graph without an eager call first)."""
    _check(lib().fno_init(), "fno_init")


def _check(status: int, where: str) -> None:
    if status != 0:
        msg = fno_status_string(status)
        if status == -7:
            msg += f" (hipError {lib().fno_last_hip_error()})"
        raise FnoError(status, where, msg)


def _torch():
    import torch
    return torch


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, ndim, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _conv2d_args(x, w, mx, my, out):
    torch = _torch()
    _need(x, torch.float32, 4, "x")
    _need(w, torch.complex64, 5, "w")
    b, cin, h, wd = x.shape
    if tuple(w.shape[:4]) != (2, mx, my, cin):
        raise ValueError(f"w has shape {tuple(w.shape)}, expected (2, {mx}, {my}, {cin}, Cout)")
    cout = w.shape[4]
    if out is None:
        out = torch.empty((b, cout, h, wd), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, 4, "out")
    if tuple(out.shape) != (b, cout, h, wd):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(b, cout, h, wd)}")
    if w.device != x.device or out.device != x.device:
        raise ValueError("x, w and out must be on the same device")
    return out, (b, cin, cout, h, wd)


def _conv1d_args(x, w, modes, out):
    torch = _torch()
    _need(x, torch.float32, 3, "x")
    _need(w, torch.complex64, 3, "w")
    b, cin, n = x.shape
    if tuple(w.shape[:2]) != (modes, cin):
        raise ValueError(f"w has shape {tuple(w.shape)}, expected ({modes}, {cin}, Cout)")
    cout = w.shape[2]
    if out is None:
        out = torch.empty((b, cout, n), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, 3, "out")
    if tuple(out.shape) != (b, cout, n):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(b, cout, n)}")
    if w.device != x.device or out.device != x.device:
        raise ValueError("x, w and out must be on the same device")
    return out, (b, cin, cout, n)


_SAME_DEVICE = contextlib.nullcontext()


def _on_device(t):
    """Make t's device current for the call (a no-op when it already is,
    which keeps the per-call host cost of small problems down)."""
    torch = _torch()
    idx = t.device.index
    if idx is None or idx == torch.cuda.current_device():
        return _SAME_DEVICE
    return torch.cuda.device(t.device)


def fno_spectral_conv2d(x, w, mx: int, my: int, out=None):
    """2D spectral convolution; returns out[B,Cout,H,W] (fastest schedule)."""
    out, (b, cin, cout, h, wd) = _conv2d_args(x, w, mx, my, out)
    with _on_device(x):
        _check(lib().fno_spectral_conv2d(_ptr(x), _ptr(w), _ptr(out), b, cin, cout, h, wd, mx, my,
                                         _stream_ptr(x.device)), "fno_spectral_conv2d")
    return out


def _epilogue_args(x, bias, branch, out, cout):
    torch = _torch()
    if bias is not None:
        _need(bias, torch.float32, 1, "bias")
        if bias.shape[0] != cout or bias.device != x.device:
            raise ValueError(f"bias must be [{cout}] on {x.device}")
    if branch is not None:
        _need(branch, torch.float32, out.dim(), "branch")
        if branch.shape != out.shape or branch.device != x.device:
            raise ValueError(f"branch must have the output's shape {tuple(out.shape)} on {x.device}")
    nullp = ctypes.c_void_p(0)
    return (_ptr(bias) if bias is not None else nullp), (_ptr(branch) if branch is not None else nullp)


def fno_spectral_conv2d_gelu(x, w, mx: int, my: int, bias=None, branch=None, branch_after: bool = False, out=None):
    """Spectral convolution with the fused layer tail: out = gelu(conv + bias[o] + branch),
    or gelu(conv + bias[o]) + branch with branch_after; bias [Cout] and branch (the output's
    shape) are optional; gelu is the exact erf form."""
    out, (b, cin, cout, h, wd) = _conv2d_args(x, w, mx, my, out)
    pb, pr = _epilogue_args(x, bias, branch, out, cout)
    with _on_device(x):
        _check(lib().fno_spectral_conv2d_gelu(_ptr(x), _ptr(w), pb, pr, _ptr(out), b, cin, cout, h, wd, mx, my,
                                              int(bool(branch_after)), _stream_ptr(x.device)),
               "fno_spectral_conv2d_gelu")
    return out


def fno_spectral_conv1d_gelu(x, w, modes: int, bias=None, branch=None, branch_after: bool = False, out=None):
    """The 1D form of fno_spectral_conv2d_gelu (branch [B,Cout,N])."""
    out, (b, cin, cout, n) = _conv1d_args(x, w, modes, out)
    pb, pr = _epilogue_args(x, bias, branch, out, cout)
    with _on_device(x):
        _check(lib().fno_spectral_conv1d_gelu(_ptr(x), _ptr(w), pb, pr, _ptr(out), b, cin, cout, n, modes,
                                              int(bool(branch_after)), _stream_ptr(x.device)),
               "fno_spectral_conv1d_gelu")
    return out


def fno_spectral_filter2d(x, mask, mx: int, my: int, out=None):
    """Diagonal global filter: out[B,C,H,W] = C2R(truncate(R2C(x)) * mask), mask [2,mx,my,C] c64."""
    torch = _torch()
    _need(x, torch.float32, 4, "x")
    _need(mask, torch.complex64, 4, "mask")
    b, c, h, wd = x.shape
    if tuple(mask.shape) != (2, mx, my, c):
        raise ValueError(f"mask has shape {tuple(mask.shape)}, expected (2, {mx}, {my}, {c})")
    if out is None:
        out = torch.empty_like(x)
    _need(out, torch.float32, 4, "out")
    if out.shape != x.shape or mask.device != x.device or out.device != x.device:
        raise ValueError("mask and out must be on x's device, out of x's shape")
    with _on_device(x):
        _check(lib().fno_spectral_filter2d(_ptr(x), _ptr(mask), _ptr(out), b, c, h, wd, mx, my,
                                           _stream_ptr(x.device)), "fno_spectral_filter2d")
    return out


def fno_spectral_filter1d(x, mask, modes: int, out=None):
    """The 1D form: x [B,C,N], mask [modes,C] c64."""
    torch = _torch()
    _need(x, torch.float32, 3, "x")
    _need(mask, torch.complex64, 2, "mask")
    b, c, n = x.shape
    if tuple(mask.shape) != (modes, c):
        raise ValueError(f"mask has shape {tuple(mask.shape)}, expected ({modes}, {c})")
    if out is None:
        out = torch.empty_like(x)
    _need(out, torch.float32, 3, "out")
    if out.shape != x.shape or mask.device != x.device or out.device != x.device:
        raise ValueError("mask and out must be on x's device, out of x's shape")
    with _on_device(x):
        _check(lib().fno_spectral_filter1d(_ptr(x), _ptr(mask), _ptr(out), b, c, n, modes, _stream_ptr(x.device)),
               "fno_spectral_filter1d")
    return out


def fno_linear_conv_length(n: int, k: int) -> int:
    """Padded transform length of the linear convolution of n samples with a k-tap kernel."""
    return int(lib().fno_linear_conv_length(int(n), int(k)))


def fno_linear_conv2d_prepare(k, h: int, w: int):
    """Weight spectrum [2,PH/2,PW/2+1,Cin,Cout] c64 of kernels k [Cout,Cin,kh,kw] f32 for H x W inputs."""
    torch = _torch()
    _need(k, torch.float32, 4, "k")
    cout, cin, kh, kw = k.shape
    ph, pw = fno_linear_conv_length(h, kh), fno_linear_conv_length(w, kw)
    if not ph or not pw:
        raise ValueError("padded grid out of range")
    wspec = torch.empty((2, ph // 2, pw // 2 + 1, cin, cout), dtype=torch.complex64, device=k.device)
    with _on_device(k):
        _check(lib().fno_linear_conv2d_prepare(_ptr(k), _ptr(wspec), cin, cout, h, w, kh, kw,
                                               _stream_ptr(k.device)), "fno_linear_conv2d_prepare")
    return wspec


def fno_linear_conv2d(x, k, crop=None, out_size=None, wspec=None, out=None):
    """Linear convolution of x [B,Cin,H,W] with k [Cout,Cin,kh,kw] (sum over Cin), cropped:
    out = y[:, :, ch:ch+Ho, cw:cw+Wo] with crop = (ch, cw), out_size = (Ho, Wo); the defaults
    give the "same" output (crop ((kh-1)//2, (kw-1)//2), size H x W).  wspec (from
    fno_linear_conv2d_prepare) skips the kernel transform."""
    torch = _torch()
    _need(x, torch.float32, 4, "x")
    _need(k, torch.float32, 4, "k")
    b, cin, h, w = x.shape
    cout, cin2, kh, kw = k.shape
    if cin2 != cin:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected (Cout, {cin}, kh, kw)")
    ch, cw = crop if crop is not None else ((kh - 1) // 2, (kw - 1) // 2)
    ho, wo = out_size if out_size is not None else (h, w)
    if wspec is None:
        wspec = fno_linear_conv2d_prepare(k, h, w)
    if out is None:
        out = torch.empty((b, cout, ho, wo), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, 4, "out")
    if tuple(out.shape) != (b, cout, ho, wo):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(b, cout, ho, wo)}")
    with _on_device(x):
        _check(lib().fno_linear_conv2d(_ptr(x), _ptr(wspec), _ptr(out), b, cin, cout, h, w, kh, kw, ch, cw, ho, wo,
                                       _stream_ptr(x.device)), "fno_linear_conv2d")
    return out


def fno_linear_conv1d_prepare(k, n: int):
    """Weight spectrum [PN/2+1,Cin,Cout] c64 of kernels k [Cout,Cin,K] f32 for length-n inputs."""
    torch = _torch()
    _need(k, torch.float32, 3, "k")
    cout, cin, kk = k.shape
    pn = fno_linear_conv_length(n, kk)
    if not pn:
        raise ValueError("padded length out of range")
    wspec = torch.empty((pn // 2 + 1, cin, cout), dtype=torch.complex64, device=k.device)
    with _on_device(k):
        _check(lib().fno_linear_conv1d_prepare(_ptr(k), _ptr(wspec), cin, cout, n, kk, _stream_ptr(k.device)),
               "fno_linear_conv1d_prepare")
    return wspec


def fno_linear_conv1d(x, k, crop=None, out_len=None, wspec=None, out=None):
    """The 1D form: x [B,Cin,N], k [Cout,Cin,K]; default "same" output (crop (K-1)//2, length N)."""
    torch = _torch()
    _need(x, torch.float32, 3, "x")
    _need(k, torch.float32, 3, "k")
    b, cin, n = x.shape
    cout, cin2, kk = k.shape
    if cin2 != cin:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected (Cout, {cin}, K)")
    c0 = crop if crop is not None else (kk - 1) // 2
    no = out_len if out_len is not None else n
    if wspec is None:
        wspec = fno_linear_conv1d_prepare(k, n)
    if out is None:
        out = torch.empty((b, cout, no), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, 3, "out")
    if tuple(out.shape) != (b, cout, no):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(b, cout, no)}")
    with _on_device(x):
        _check(lib().fno_linear_conv1d(_ptr(x), _ptr(wspec), _ptr(out), b, cin, cout, n, kk, c0, no,
                                       _stream_ptr(x.device)), "fno_linear_conv1d")
    return out


def fno_spectral_conv2d_unfused(x, w, mx: int, my: int, out=None):
    """2D spectral convolution through the unfused stage kernels (ablation)."""
    out, (b, cin, cout, h, wd) = _conv2d_args(x, w, mx, my, out)
    with _on_device(x):
        _check(lib().fno_spectral_conv2d_unfused(_ptr(x), _ptr(w), _ptr(out), b, cin, cout, h, wd, mx, my,
                                                 _stream_ptr(x.device)), "fno_spectral_conv2d_unfused")
    return out


def fno_workspace_size_2d(B, Cin, Cout, H, W, mx, my) -> int:
    return int(lib().fno_workspace_size_2d(B, Cin, Cout, H, W, mx, my))


def fno_workspace_size_1d(B, Cin, Cout, N, modes) -> int:
    return int(lib().fno_workspace_size_1d(B, Cin, Cout, N, modes))


def fno_spectral_conv2d_ws(x, w, mx: int, my: int, workspace, out=None):
    """2D spectral convolution with caller-owned scratch (a uint8 CUDA tensor)."""
    out, (b, cin, cout, h, wd) = _conv2d_args(x, w, mx, my, out)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with _on_device(x):
        _check(lib().fno_spectral_conv2d_ws(_ptr(x), _ptr(w), _ptr(out), b, cin, cout, h, wd, mx, my,
                                            ws_ptr, ws_bytes, _stream_ptr(x.device)), "fno_spectral_conv2d_ws")
    return out


def fno_spectral_conv2d_noalloc(x, w, mx: int, my: int, out=None):
    """2D spectral convolution whose scratch is the library's fixed device
    array (no allocation inside the call; fno_init must have run on the
    device).  `out` must be given by callers that cannot allocate."""
    out, (b, cin, cout, h, wd) = _conv2d_args(x, w, mx, my, out)
    with _on_device(x):
        _check(lib().fno_spectral_conv2d_noalloc(_ptr(x), _ptr(w), _ptr(out), b, cin, cout, h, wd, mx, my,
                                                 _stream_ptr(x.device)), "fno_spectral_conv2d_noalloc")
    return out


def fno_noalloc_scratch_bytes() -> int:
    """Bytes of the fixed device array fno_spectral_conv2d_noalloc uses."""
    return int(lib().fno_noalloc_scratch_bytes())


def fno_spectral_conv1d(x, w, modes: int, out=None):
    """1D spectral convolution along the last axis; returns out[B,Cout,N]."""
    out, (b, cin, cout, n) = _conv1d_args(x, w, modes, out)
    with _on_device(x):
        _check(lib().fno_spectral_conv1d(_ptr(x), _ptr(w), _ptr(out), b, cin, cout, n, modes,
                                         _stream_ptr(x.device)), "fno_spectral_conv1d")
    return out


def fno_spectral_conv1d_unfused(x, w, modes: int, out=None):
    out, (b, cin, cout, n) = _conv1d_args(x, w, modes, out)
    with _on_device(x):
        _check(lib().fno_spectral_conv1d_unfused(_ptr(x), _ptr(w), _ptr(out), b, cin, cout, n, modes,
                                                 _stream_ptr(x.device)), "fno_spectral_conv1d_unfused")
    return out


def fno_spectral_conv1d_ws(x, w, modes: int, workspace, out=None):
    out, (b, cin, cout, n) = _conv1d_args(x, w, modes, out)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with _on_device(x):
        _check(lib().fno_spectral_conv1d_ws(_ptr(x), _ptr(w), _ptr(out), b, cin, cout, n, modes,
                                            ws_ptr, ws_bytes, _stream_ptr(x.device)), "fno_spectral_conv1d_ws")
    return out


def _grad_outputs(x, w, grad_out, need_x, need_w, out_shape, grad_x, grad_w):
    torch = _torch()
    if not (need_x or need_w):
        raise ValueError("ask for at least one of the two gradients")
    _need(grad_out, torch.float32, x.dim(), "grad_out")
    if tuple(grad_out.shape) != out_shape:
        raise ValueError(f"grad_out has shape {tuple(grad_out.shape)}, expected {out_shape}")
    if grad_out.device != x.device:
        raise ValueError("grad_out must be on the device of x")

    def target(given, like, name):
        if given is None:
            return torch.empty_like(like)
        _need(given, like.dtype, like.dim(), name)
        if given.shape != like.shape or given.device != like.device:
            raise ValueError(f"{name} must match {tuple(like.shape)} on {like.device}")
        return given

    gx = target(grad_x, x, "grad_x") if need_x else None
    gw = target(grad_w, w, "grad_w") if need_w else None
    return gx, gw


def fno_spectral_conv2d_backward(x, w, grad_out, mx: int, my: int, need_x: bool = True, need_w: bool = True,
                                 grad_x=None, grad_w=None):
    """Gradients (grad_x[B,Cin,H,W] f32, grad_w[2,mx,my,Cin,Cout] c64) of a real loss
    through fno_spectral_conv2d, given grad_out = dL/dout; grad_w = dL/dRe w + i dL/dIm w.
    A gradient not asked for is returned as None; grad_x / grad_w, when given,
    are written in place of new tensors."""
    _, (b, cin, cout, h, wd) = _conv2d_args(x, w, mx, my, grad_out)
    gx, gw = _grad_outputs(x, w, grad_out, need_x, need_w, (b, cout, h, wd), grad_x, grad_w)
    nullp = ctypes.c_void_p(0)
    with _on_device(x):
        _check(lib().fno_spectral_conv2d_backward(_ptr(x), _ptr(w), _ptr(grad_out),
                                                  _ptr(gx) if gx is not None else nullp,
                                                  _ptr(gw) if gw is not None else nullp,
                                                  b, cin, cout, h, wd, mx, my, _stream_ptr(x.device)),
               "fno_spectral_conv2d_backward")
    return gx, gw


def fno_spectral_conv1d_backward(x, w, grad_out, modes: int, need_x: bool = True, need_w: bool = True,
                                 grad_x=None, grad_w=None):
    """Gradients (grad_x[B,Cin,N] f32, grad_w[modes,Cin,Cout] c64) through fno_spectral_conv1d."""
    _, (b, cin, cout, n) = _conv1d_args(x, w, modes, grad_out)
    gx, gw = _grad_outputs(x, w, grad_out, need_x, need_w, (b, cout, n), grad_x, grad_w)
    nullp = ctypes.c_void_p(0)
    with _on_device(x):
        _check(lib().fno_spectral_conv1d_backward(_ptr(x), _ptr(w), _ptr(grad_out),
                                                  _ptr(gx) if gx is not None else nullp,
                                                  _ptr(gw) if gw is not None else nullp,
                                                  b, cin, cout, n, modes, _stream_ptr(x.device)),
               "fno_spectral_conv1d_backward")
    return gx, gw


def fno_forward2d(x, mx: int, my: int, xh=None):
    """Truncated ortho spectrum xh[B,C,2,mx,my] (complex64) of x[B,C,H,W]."""
    torch = _torch()
    _need(x, torch.float32, 4, "x")
    b, c, h, wd = x.shape
    if xh is None:
        xh = torch.empty((b, c, 2, mx, my), dtype=torch.complex64, device=x.device)
    _need(xh, torch.complex64, 5, "xh")
    if tuple(xh.shape) != (b, c, 2, mx, my):
        raise ValueError(f"xh has shape {tuple(xh.shape)}, expected {(b, c, 2, mx, my)}")
    with _on_device(x):
        _check(lib().fno_forward2d(_ptr(x), _ptr(xh), b, c, h, wd, mx, my, _stream_ptr(x.device)),
               "fno_forward2d")
    return xh


def fno_inverse2d(yh, h: int, w: int, out=None):
    """out[B,C,H,W] from a truncated spectrum yh[B,C,2,mx,my] (zero-fill + ortho C2R)."""
    torch = _torch()
    _need(yh, torch.complex64, 5, "yh")
    b, c, _, mx, my = yh.shape
    if out is None:
        out = torch.empty((b, c, h, w), dtype=torch.float32, device=yh.device)
    _need(out, torch.float32, 4, "out")
    if tuple(out.shape) != (b, c, h, w):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(b, c, h, w)}")
    with _on_device(yh):
        _check(lib().fno_inverse2d(_ptr(yh), _ptr(out), b, c, h, w, mx, my, _stream_ptr(yh.device)),
               "fno_inverse2d")
    return out


def fno_forward1d(x, modes: int, xh=None):
    torch = _torch()
    _need(x, torch.float32, 3, "x")
    b, c, n = x.shape
    if xh is None:
        xh = torch.empty((b, c, modes), dtype=torch.complex64, device=x.device)
    _need(xh, torch.complex64, 3, "xh")
    with _on_device(x):
        _check(lib().fno_forward1d(_ptr(x), _ptr(xh), b, c, n, modes, _stream_ptr(x.device)), "fno_forward1d")
    return xh


def fno_inverse1d(yh, n: int, out=None):
    torch = _torch()
    _need(yh, torch.complex64, 3, "yh")
    b, c, modes = yh.shape
    if out is None:
        out = torch.empty((b, c, n), dtype=torch.float32, device=yh.device)
    _need(out, torch.float32, 3, "out")
    with _on_device(yh):
        _check(lib().fno_inverse1d(_ptr(yh), _ptr(out), b, c, n, modes, _stream_ptr(yh.device)), "fno_inverse1d")
    return out


def fno_mix(xh, w, yh=None):
    """yh[b,o,m] = sum_i xh[b,i,m] w[m,i,o]; xh [B,Cin,...modes], w [...modes,Cin,Cout] complex64."""
    torch = _torch()
    if xh.dtype != torch.complex64 or w.dtype != torch.complex64:
        raise TypeError("xh and w must be complex64")
    if not (xh.is_contiguous() and w.is_contiguous()):
        raise ValueError("xh and w must be contiguous")
    b, cin = xh.shape[0], xh.shape[1]
    m = xh[0, 0].numel()
    cout = w.shape[-1]
    if w.shape[-2] != cin or w.numel() != m * cin * cout:
        raise ValueError(f"w has shape {tuple(w.shape)}, incompatible with xh {tuple(xh.shape)}")
    if yh is None:
        yh = torch.empty((b, cout) + tuple(xh.shape[2:]), dtype=torch.complex64, device=xh.device)
    with _on_device(xh):
        _check(lib().fno_mix(_ptr(xh), _ptr(w), _ptr(yh), b, cin, cout, m, _stream_ptr(xh.device)), "fno_mix")
    return yh


def fno_set_timing_events(events):
    """Launch kernel k of later calls on this thread with events[2k] and
    events[2k+1] (torch.cuda.Event, already recorded once so that the HIP
    event exists) as its start and stop events (see include/fno.h); pass None
    to stop.  The list must stay alive while recording is on."""
    global _timing_keepalive
    if events is None:
        _timing_keepalive = None
        _check(lib().fno_set_timing_events(None, 0), "fno_set_timing_events")
        return
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    _timing_keepalive = (arr, events)
    _check(lib().fno_set_timing_events(arr, len(events)), "fno_set_timing_events")


_timing_keepalive = None


def fno_last_kernels():
    """Names of the kernels the last successful call on this thread launched."""
    n = lib().fno_last_kernel_count()
    return [lib().fno_last_kernel_name(i).decode() for i in range(n)]
