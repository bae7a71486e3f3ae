// Host-side internal interface between the C ABI (fno_abi.hip) and the kernel
// launchers.  Not part of the public API.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace fno {

struct Shape2d {
    int64_t B, Cin, Cout;
    int H, W, mx, my;
    int log2H, log2W;
};

struct Shape1d {
    int64_t B, Cin, Cout;
    int N, modes, log2N;
};

// Address of truncated-spectrum entry (b, c, m), in complex elements:
//   b * sb + c * sc + (m / 8) * st + (m % 8)
// Canonical [B][C][M]: sb = C*M, sc = M, st = 8.
// Tiled [B][ceil(M/8)][C][8] (8 modes of one (b, c) form a 64-byte chunk).
struct SpecLayout {
    int64_t sb, sc, st;
    int C;
};

// Events the next kernel launch carries (set by the per-kernel timing
// recorder of the C ABI, both null otherwise).  Taking them clears them.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents take_launch_events();

// Every kernel is launched through here: with per-kernel timing on, the
// launch itself carries the events, which then take the kernel's own start
// and end timestamps (no marker packets between dependent kernels).
template <typename K, typename... Args>
hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
    const LaunchEvents ev = take_launch_events();
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, s, ev.start, ev.stop, 0u, args...);
    return hipGetLastError();
}

// True while `s` is being captured into a HIP graph (nothing may be
// allocated, freed or copied synchronously then).
inline bool stream_capturing(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return cs != hipStreamCaptureStatusNone;
}

inline SpecLayout canonical_layout(int64_t C, int64_t M) { return SpecLayout{C * M, M, 8, (int)C}; }
// The canonical layout with each channel's M modes padded to a whole number
// of 8-mode runs (channel stride M rounded up to 8); the padding slots hold
// no modes (the mix may write there).
inline SpecLayout padded_layout(int64_t C, int64_t M) {
    const int64_t mp = (M + 7) / 8 * 8;
    return SpecLayout{C * mp, mp, 8, (int)C};
}
inline SpecLayout tiled_layout(int64_t C, int64_t M) {
    const int64_t nt = (M + 7) / 8;
    return SpecLayout{nt * C * 8, 8, C * 8, (int)C};
}
// Complex elements a spectrum of B batch items spans in either layout.
inline int64_t layout_elems(const SpecLayout& l, int64_t B) { return B * l.sb; }

// ---- fused output epilogue of the inverse transforms ------------------------
// The FFT blog's fused operator (sections 5.1-5.2) activates the C2R output
// with GELU and adds a second, time-domain branch in the kernel that writes
// the output (section 6.2: fuse what follows the C2R).  With `on` set, each
// output value v of channel c becomes
//   gelu(v + bias[c] + branch)     (branch_after == 0: the FNO-layer form), or
//   gelu(v + bias[c]) + branch     (branch_after == 1: the blog's order),
// branch read at the output's own index (same shape as the output), a null
// bias or branch reads as zero, gelu(u) = u (1 + erf(u / sqrt 2)) / 2.  The
// channel of output row r (rows of the kernel's row length) is
// (r / rows_per_chan) % cout; the per-image kernels pass their image index
// with rows_per_chan = 1.  Row and image indices fit 32 bits on this path
// (checked by the caller).
struct Epilogue {
    bool on = false;
    const float* branch = nullptr;
    const float* bias = nullptr;
    uint32_t rows_per_chan = 1;
    uint32_t cout = 1;
    int branch_after = 0;
};

// gelu(u) = u Phi(u) = (u / 2) erfc(-u / sqrt 2), with erfc from the
// Chebyshev fit of Numerical Recipes (2nd ed., section 6.2, "erfcc":
// fractional error below 1.2e-7 everywhere), written without branches so
// that the epilogue stays straight-line code:
//   t = 1 / (1 + |z| / 2),
//   erfc(|z|) = t exp(-z^2 - 1.26551223 + t (1.00002368 + t (0.37409196 + ...))),
//   erfc(-|z|) = 2 - erfc(|z|).
__device__ __forceinline__ float epi_erfc(float z) {
    const float a = fabsf(z);
    const float t = __frcp_rn(fmaf(0.5f, a, 1.0f));
    float p = 0.17087277f;
    p = fmaf(p, t, -0.82215223f);
    p = fmaf(p, t, 1.48851587f);
    p = fmaf(p, t, -1.13520398f);
    p = fmaf(p, t, 0.27886807f);
    p = fmaf(p, t, -0.18628806f);
    p = fmaf(p, t, 0.09678418f);
    p = fmaf(p, t, 0.37409196f);
    p = fmaf(p, t, 1.00002368f);
    p = fmaf(p, t, -1.26551223f);
    const float r = t * __expf(fmaf(-a, a, p));
    return z >= 0.0f ? r : 2.0f - r;
}
__device__ __forceinline__ float epi_gelu(float u) { return 0.5f * u * epi_erfc(-0.707106781186547524f * u); }
// bias of output row (or image) r, read through a buffer resource (an empty
// range for a null bias reads zero), so that no branch enters the kernel
__device__ __forceinline__ float epi_bias(const Epilogue& e, uint32_t r) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(e.bias, e.bias ? e.cout * 4u : 0u);
    const uint32_t ch = (r / e.rows_per_chan) % e.cout;
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(ch * 4u), 0, 0));
}
__device__ __forceinline__ float epi_apply(const Epilogue& e, float v, float bias, float br) {
    const float pre = e.branch_after ? 0.0f : br;
    return epi_gelu(v + bias + pre) + (br - pre);
}

// ---- fused small-grid transforms (fno_small2d.hip), H, W in [8, 128] --------
bool small2d_supported(int log2H, int log2W, int my);
// The whole 2D call in one kernel for small problems (grids of at most 1024
// points, 8..128 per side, at most 8 channels in and out): one workgroup per
// batch item, the truncated spectra in LDS; scale = (H W)^-1/2, applied on
// both transforms.
bool conv2d_small_fused_supported(int64_t B, int64_t Cin, int64_t Cout, int log2H, int log2W, int mx, int my);
hipError_t launch_conv2d_small_fused(const float* x, const float2* w, float* out, int64_t B, int64_t Cin, int64_t Cout,
                                     int log2H, int log2W, int mx, int my, float scale, const float2* tw,
                                     hipStream_t s);
hipError_t launch_fwd2d_small(const float* x, float2* xh, const SpecLayout& lay, int64_t nimg, int log2H, int log2W,
                              int mx, int my, float scale, const float2* tw, hipStream_t s);
hipError_t launch_inv2d_small(const float2* yh, float* out, const SpecLayout& lay, int64_t nimg, int log2H,
                              int log2W, int mx, int my, float scale, const float2* tw, hipStream_t s,
                              const Epilogue& epi = Epilogue{});

// ---- 2D transforms with one real row per thread (fno_rowreg2d.hip) ---------
// H, W in {64, 128}, my <= 32; same output as launch_fwd2d_small (scaled by
// (HW)^-1/2).  Persistent grid sized from the kernel's occupancy.
bool rowreg2d_supported(int log2H, int log2W, int mx, int my, const SpecLayout& lay);
// mask_t (optional): the diagonal filter applied on the way out,
// xh(b, c, m) *= mask_t[c][m] (the mask transposed channel-major)
hipError_t launch_fwd2d_rowreg(const float* x, float2* xh, const SpecLayout& lay, int64_t nimg, int log2H,
                               int log2W, int mx, int my, const float2* tw, hipStream_t s,
                               const float2* mask = nullptr);
// and its inverse: truncated spectrum -> real image, same shapes and scale
hipError_t launch_inv2d_rowreg(const float2* yh, float* out, const SpecLayout& lay, int64_t nimg, int log2H,
                               int log2W, int mx, int my, const float2* tw, hipStream_t s,
                               const Epilogue& epi = Epilogue{});

// ---- channel mix on MFMA (fno_mix.hip) --------------------------------------
// yh(b, o, m) = sum_i xh(b, i, m) * w[m][i][o], spectra addressed by layouts.
// Needs an even Cout, a 16-byte aligned w (float4 weight pairs) and Cin <= 128.
// adjoint: yh(b, o, m) = sum_i xh(b, i, m) * conj(w[m][o][i]) instead (the
// weight of the forward layer, read transposed); needs an even Cin, Cin <=
// 128, a 16-byte aligned w and spectra with whole, aligned 8-mode runs
// (mix_mfma_adjoint_supported).
bool mix_mfma_supported(int64_t Cin, int64_t Cout, const void* w);
bool mix_mfma_adjoint_supported(const float2* xh, const SpecLayout& lx, const float2* w, const float2* yh,
                                const SpecLayout& ly, int64_t Cin, int64_t M);
hipError_t launch_mix_mfma(const float2* xh, const SpecLayout& lx, const float2* w, float2* yh,
                           const SpecLayout& ly, int64_t B, int64_t Cin, int64_t Cout, int64_t M, hipStream_t s,
                           bool adjoint = false);

// ---- per-image transforms of 128- to 512-row grids (fno_short2d.hip) ---------
// 128 x 256, or H in {256, 512} and W in {128, 256, 512}; my <= 32 (16 at
// H = 512), 2 mx a multiple of 16 (at most 128, 64 at H = 128):
// the row and column passes of one image in one workgroup, the row spectrum
// in LDS.  Forward: x [nimg][H][W] -> the canonical spectrum
// xh [nimg][2 mx][my] (kept kx rows, mode q my + ky), scaled by scale.
bool short2d_supported(int log2H, int log2W, int mx, int my);
// whether the one-kernel form pays for nimg images of 2^log2H rows of
// 2^log2W points (enough images for the CUs; with 128-point rows, at most
// one per CU, one per two CUs at 512 rows)
bool short2d_pays(int64_t nimg, int log2H, int log2W);
hipError_t launch_fwd2d_short(const float* x, float2* xh, int64_t nimg, int log2H, int log2W, int mx, int my,
                              float scale, const float2* tw, hipStream_t s);
// Inverse: the canonical spectrum yh [nimg][2 mx][my] -> out [nimg][H][W]
// times scale; epi: the fused layer epilogue (rows_per_chan = H).
hipError_t launch_inv2d_short(const float2* yh, float* out, int64_t nimg, int log2H, int log2W, int mx, int my,
                              float scale, const float2* tw, hipStream_t s, const Epilogue& epi);

// ---- pruned row transforms (fno_rows_pruned.hip) ----------------------------
// Rows of W = 2^log2W real points, W in [64, 4096], bins ky < my <= 64
// (my <= 32 at W = 64):
// same contract as launch_rows_fwd / launch_rows_inv below, which use them
// whenever rows_pruned_supported holds.
bool rows_pruned_supported(int log2W, int my);
hipError_t launch_rows_fwd_pruned(const float* x, float2* y, int64_t nrows, int log2W, int my, int y_ld, float scale,
                                  const float2* tw, hipStream_t s);
hipError_t launch_rows_inv_pruned(const float2* y, float* out, int64_t nrows, int log2W, int my, int y_ld,
                                  float scale, const float2* tw, hipStream_t s, const Epilogue& epi = Epilogue{});

// ---- pruned column transforms (fno_cols_pruned.hip) --------------------------
// H in [256, 2048], 2 mx <= 128 and a multiple of H / 64, my <= 64: same
// contract as launch_cols_fwd / launch_cols_inv below, which use them
// whenever cols_pruned_supported holds.
bool cols_pruned_supported(int log2H, int mx, int my);
hipError_t launch_cols_fwd_pruned(const float2* r, float2* xh, int64_t nimg, int log2H, int mx, int my, float scale,
                                  const float2* tw, hipStream_t s);
hipError_t launch_cols_inv_pruned(const float2* yh, float2* r, int64_t nimg, int log2H, int mx, int my,
                                  const float2* tw, hipStream_t s);

// ---- generic stage launchers (fno_generic.hip) -------------------------------
// All return hipSuccess or the launch error.  `tw` is the device twiddle table.

// Rows of length W (real) -> bins ky < my, row-major [nrows][y_ld], times scale.
hipError_t launch_rows_fwd(const float* x, float2* y, int64_t nrows, int log2W, int my, int y_ld,
                           float scale, const float2* tw, hipStream_t s);
// R[nimg][H][my] -> xh[nimg][2][mx][my] (kept kx only), times scale.
hipError_t launch_cols_fwd(const float2* r, float2* xh, int64_t nimg, int log2H, int mx, int my,
                           float scale, const float2* tw, hipStream_t s);
// Per-mode channel mix, VALU: yh(b, o, m) = sum_i xh(b, i, m) w[m][i][o].
hipError_t launch_mix_valu(const float2* xh, const SpecLayout& lx, const float2* w, float2* yh,
                           const SpecLayout& ly, int64_t B, int64_t Cin, int64_t Cout, int64_t M, hipStream_t s);
// yh[nimg][2][mx][my] -> zero-filled column inverse -> R'[nimg][H][my].
hipError_t launch_cols_inv(const float2* yh, float2* r, int64_t nimg, int log2H, int mx, int my,
                           const float2* tw, hipStream_t s);
// R'[nrows][y_ld] (bins ky < my) -> C2R rows of length W, times scale.
hipError_t launch_rows_inv(const float2* y, float* out, int64_t nrows, int log2W, int my, int y_ld,
                           float scale, const float2* tw, hipStream_t s, const Epilogue& epi = Epilogue{});

// ---- diagonal global filter (fno_filter.hip) --------------------------------
// yh(b, c, m) = xh(b, c, m) * mask[m][c], both spectra in layout `lay`
// (tiled or canonical).
bool mix_diag_supported(const SpecLayout& lay, int64_t M);
// mt[c][m] = mask[m][c] (M modes, C channels)
hipError_t launch_mask_transpose(const float2* mask, float2* mt, int64_t M, int64_t C, hipStream_t s);
hipError_t launch_mix_diag(const float2* xh, float2* yh, const SpecLayout& lay, const float2* mask, int64_t B,
                           int64_t C, int64_t M, hipStream_t s);

// ---- mixed-radix stage kernels (fno_mixed.hip) -----------------------------
// Same contracts as launch_rows_fwd / launch_cols_fwd / launch_cols_inv /
// launch_rows_inv, for 7-smooth lengths 2..4096 given as lengths (W, H).
// A RowWindow makes the rows those of images of ph rows of which only a
// window is stored: forward, x holds each image's top-left h x w corner
// (the rest reads as zero); inverse, only rows [h0, h0+h) x columns
// [w0, w0+w) are written, packed (no epilogue with a window).
struct RowWindow {
    int ph, h, w, h0, w0;
};
bool mixed_supported(int n);
// 7-smooth lengths up to 8192 for the row kernels alone (no epilogue beyond
// 4096 points): the rows of a zero-padded linear convolution.
bool mixed_row_supported(int n);
hipError_t launch_rows_fwd_mr(const float* x, float2* y, int64_t nrows, int W, int my, int y_ld, float scale,
                              hipStream_t s, const RowWindow* window = nullptr);
// layout: where mode m = q my + ky of image img = b C + c sits in the
// spectrum (default: image after image, 2 mx my modes each)
hipError_t launch_cols_fwd_mr(const float2* r, float2* xh, int64_t nimg, int H, int mx, int my, float scale,
                              hipStream_t s, const SpecLayout* layout = nullptr);
hipError_t launch_cols_inv_mr(const float2* yh, float2* r, int64_t nimg, int H, int mx, int my, hipStream_t s,
                              const SpecLayout* layout = nullptr);
hipError_t launch_rows_inv_mr(const float2* y, float* out, int64_t nrows, int W, int my, int y_ld, float scale,
                              hipStream_t s, const Epilogue& epi = Epilogue{}, const RowWindow* window = nullptr);

// ---- zero-padded linear convolution helpers (fno_linconv.hip) ---------------
// dst[img][PH][PW] = src[img][H][W] zero-padded (bottom and right).
hipError_t launch_pad2d(const float* src, float* dst, int64_t nimg, int H, int W, int PH, int PW, hipStream_t s);
// w[m][i][o] = scale * kh[o Cin + i][m] (kh canonical spectra of the kernels).
hipError_t launch_spec_to_weight(const float2* kh, float2* w, int64_t M, int64_t Cin, int64_t Cout, float scale,
                                 hipStream_t s);

// ---- backward pass (fno_backward.hip) ---------------------------------------
// wt[m][o][i] = conj(w[m][i][o]) for M modes.
hipError_t launch_weight_adjoint(const float2* w, float2* wt, int64_t M, int64_t Cin, int64_t Cout, hipStream_t s);
// gw[m][i][o] = c_m sum_b conj(xh(b, i, m)) gh(b, o, m), c_m = 1 when
// ky = m mod my is 0 or nyq, 2 otherwise (spectra addressed by layouts).
// When the batch is split (*splits > 1 on return) the partial sums are left
// in ws (weight_grad_workspace bytes) and launch_weight_grad_reduce must
// follow to write gw.
size_t weight_grad_workspace(int64_t B, int64_t Cin, int64_t Cout, int64_t M);
hipError_t launch_weight_grad(const float2* xh, const SpecLayout& lx, const float2* gh, const SpecLayout& lg,
                              float2* gw, int64_t B, int64_t Cin, int64_t Cout, int64_t M, int my, int nyq, void* ws,
                              size_t ws_bytes, int* splits, hipStream_t s);
hipError_t launch_weight_grad_reduce(const void* ws, float2* gw, int64_t Cin, int64_t Cout, int64_t M, int splits,
                                     int my, int nyq, hipStream_t s);

}  // namespace fno
