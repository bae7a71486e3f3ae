// Generic stage kernels of the spectral convolution: any power-of-two H, W up
// to 4096, any mode counts.  Each stage is one kernel; the spectra between
// stages live in device memory.  These are the building blocks of the
// unfused schedule and the fallback for shapes without a specialised kernel.
//
// Stages (TurboFNO blog, sections 2.1-2.2; FFT blog, sections 2.1-2.2):
//   rows_fwd  real rows -> half-spectrum bins ky < my   (two real rows share
//             one complex transform: z = a + i b, A[k] = (Z[k] + conj Z[-k])/2,
//             B[k] = (Z[k] - conj Z[-k]) / 2i)
//   cols_fwd  complex columns along H -> kept kx in [0,mx) u [H-mx,H)
//   mix       per-mode Cin -> Cout complex contraction
//   cols_inv  zero-filled complex columns -> inverse along H
//   rows_inv  half spectrum bins ky < my -> real rows (C2R; Im of the DC and
//             Nyquist bins dropped; two rows per complex transform)
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kThreads = 256;

template <int LOG2W>
__global__ __launch_bounds__(kThreads) void k_rows_fwd(const float* __restrict__ x, float2* __restrict__ y,
                                                      int64_t nrows, int my, int y_ld, float scale,
                                                      const float2* __restrict__ tw) {
    constexpr int W = 1 << LOG2W;
    constexpr int P = W >= kLdsElems ? 1 : kLdsElems / W;   // complex rows (real row pairs) per block
    __shared__ float2 buf[2][kLdsElems];
    const int tid = threadIdx.x;
    const int64_t npairs = (nrows + 1) / 2;
    const int64_t pair0 = (int64_t)blockIdx.x * P;
    const int prows = (int)(npairs - pair0 < P ? npairs - pair0 : P);

    for (int e = tid; e < prows * W; e += kThreads) {
        const int pr = e >> LOG2W;
        const int n = e & (W - 1);
        const int64_t ra = 2 * (pair0 + pr);
        const float a = x[ra * W + n];
        const float b = (ra + 1 < nrows) ? x[(ra + 1) * W + n] : 0.0f;
        buf[0][pr * W + n] = make_float2(a, b);
    }
    __syncthreads();
    const float2* res = fft_rows_lds<LOG2W, -1>(buf[0], buf[1], prows, W, tw, tid, kThreads);

    for (int e = tid; e < prows * my; e += kThreads) {
        const int pr = e / my;
        const int k = e - pr * my;
        const float2 zk = res[pr * W + k];
        const float2 zm = res[pr * W + ((W - k) & (W - 1))];
        const float2 a = make_float2(0.5f * (zk.x + zm.x), 0.5f * (zk.y - zm.y));
        const float2 b = make_float2(0.5f * (zk.y + zm.y), -0.5f * (zk.x - zm.x));
        const int64_t ra = 2 * (pair0 + pr);
        y[ra * y_ld + k] = cscale(a, scale);
        if (ra + 1 < nrows) y[(ra + 1) * y_ld + k] = cscale(b, scale);
    }
}

template <int LOG2H>
__global__ __launch_bounds__(kThreads) void k_cols_fwd(const float2* __restrict__ r, float2* __restrict__ xh,
                                                      int mx, int my, int kb, int nkb, float scale,
                                                      const float2* __restrict__ tw) {
    constexpr int H = 1 << LOG2H;
    __shared__ float2 buf[2][kLdsElems];
    const int tid = threadIdx.x;
    const int64_t img = blockIdx.x / nkb;
    const int ky0 = (int)(blockIdx.x % nkb) * kb;
    const int ncol = min(kb, my - ky0);
    const float2* src = r + img * H * my;

    for (int e = tid; e < ncol * H; e += kThreads) {
        const int h = e / ncol;
        const int c = e - h * ncol;
        buf[0][c * H + h] = src[(int64_t)h * my + ky0 + c];
    }
    __syncthreads();
    const float2* res = fft_rows_lds<LOG2H, -1>(buf[0], buf[1], ncol, H, tw, tid, kThreads);

    float2* dst = xh + img * (2 * mx) * my;
    for (int e = tid; e < 2 * mx * ncol; e += kThreads) {
        const int q = e / ncol;
        const int c = e - q * ncol;
        const int kx = q < mx ? q : H - 2 * mx + q;
        dst[(int64_t)q * my + ky0 + c] = cscale(res[c * H + kx], scale);
    }
}

template <int LOG2H>
__global__ __launch_bounds__(kThreads) void k_cols_inv(const float2* __restrict__ yh, float2* __restrict__ r,
                                                      int mx, int my, int kb, int nkb,
                                                      const float2* __restrict__ tw) {
    constexpr int H = 1 << LOG2H;
    __shared__ float2 buf[2][kLdsElems];
    const int tid = threadIdx.x;
    const int64_t img = blockIdx.x / nkb;
    const int ky0 = (int)(blockIdx.x % nkb) * kb;
    const int ncol = min(kb, my - ky0);
    const float2* src = yh + img * (2 * mx) * my;

    // zero the dropped kx, then place the kept ones (disjoint locations)
    for (int e = tid; e < ncol * H; e += kThreads) {
        const int c = e >> LOG2H;
        const int kx = e & (H - 1);
        if (kx >= mx && kx < H - mx) buf[0][c * H + kx] = make_float2(0.0f, 0.0f);
    }
    for (int e = tid; e < 2 * mx * ncol; e += kThreads) {
        const int q = e / ncol;
        const int c = e - q * ncol;
        const int kx = q < mx ? q : H - 2 * mx + q;
        buf[0][c * H + kx] = src[(int64_t)q * my + ky0 + c];
    }
    __syncthreads();
    const float2* res = fft_rows_lds<LOG2H, +1>(buf[0], buf[1], ncol, H, tw, tid, kThreads);

    float2* dst = r + img * H * my;
    for (int e = tid; e < ncol * H; e += kThreads) {
        const int h = e / ncol;
        const int c = e - h * ncol;
        dst[(int64_t)h * my + ky0 + c] = res[c * H + h];
    }
}

// EPI: the fused output epilogue (bias, GELU, second branch) on every
// output, the branch read at the same index.
template <int LOG2W, bool EPI>
__global__ __launch_bounds__(kThreads) void k_rows_inv(const float2* __restrict__ y, float* __restrict__ out,
                                                      int64_t nrows, int my, int y_ld, float scale,
                                                      const float2* __restrict__ tw, Epilogue epi) {
    constexpr int W = 1 << LOG2W;
    constexpr int P = W >= kLdsElems ? 1 : kLdsElems / W;
    __shared__ float2 buf[2][kLdsElems];
    const int tid = threadIdx.x;
    const int64_t npairs = (nrows + 1) / 2;
    const int64_t pair0 = (int64_t)blockIdx.x * P;
    const int prows = (int)(npairs - pair0 < P ? npairs - pair0 : P);

    // Z = Ya_herm + i Yb_herm, with Ya_herm[W-k] = conj Ya[k] and the imaginary
    // parts of the DC / Nyquist bins dropped.
    for (int e = tid; e < prows * W; e += kThreads) {
        const int pr = e >> LOG2W;
        const int k = e & (W - 1);
        const int kk = (k <= W / 2) ? k : W - k;
        const int64_t ra = 2 * (pair0 + pr);
        float2 z = make_float2(0.0f, 0.0f);
        if (kk < my) {
            const float2 ya = y[ra * y_ld + kk];
            const float2 yb = (ra + 1 < nrows) ? y[(ra + 1) * y_ld + kk] : make_float2(0.0f, 0.0f);
            if (kk == 0 || 2 * kk == W) {
                z = make_float2(ya.x, yb.x);
            } else if (k == kk) {
                z = make_float2(ya.x - yb.y, ya.y + yb.x);
            } else {
                z = make_float2(ya.x + yb.y, yb.x - ya.y);
            }
        }
        buf[0][pr * W + k] = z;
    }
    __syncthreads();
    const float2* res = fft_rows_lds<LOG2W, +1>(buf[0], buf[1], prows, W, tw, tid, kThreads);

    for (int e = tid; e < prows * W; e += kThreads) {
        const int pr = e >> LOG2W;
        const int n = e & (W - 1);
        const int64_t ra = 2 * (pair0 + pr);
        const float2 z = res[pr * W + n];
        if constexpr (EPI) {
            // the branch through a buffer resource (an empty range for a null
            // branch reads zero); rows 2 pair0 .. of this block
            const __amdgpu_buffer_rsrc_t rb =
                make_rsrc(epi.branch ? epi.branch + 2 * pair0 * W : nullptr,
                          epi.branch ? (uint32_t)((nrows - 2 * pair0 < 2 * P ? nrows - 2 * pair0 : 2 * P) * W * 4) : 0u);
            const uint32_t off = (uint32_t)((ra - 2 * pair0) * W + n) * 4u;
            nt_store(&out[ra * W + n], epi_apply(epi, z.x * scale, epi_bias(epi, (uint32_t)ra), buffer_load_f1(rb, off, 0)));
            if (ra + 1 < nrows)
                nt_store(&out[(ra + 1) * W + n], epi_apply(epi, z.y * scale, epi_bias(epi, (uint32_t)(ra + 1)),
                                                           buffer_load_f1(rb, off + (uint32_t)W * 4u, 0)));
        } else {
            nt_store(&out[ra * W + n], z.x * scale);
            if (ra + 1 < nrows) nt_store(&out[(ra + 1) * W + n], z.y * scale);
        }
    }
}

constexpr int kMixIC = 8;   // input channels per batch of loads

struct MixAddr {
    int64_t sb, sc, st;
    __device__ __forceinline__ int64_t at(int64_t b, int64_t c, int64_t m) const {
        return b * sb + c * sc + (m >> 3) * st + (m & 7);
    }
};

// Thread (m, o) accumulates Y_m[b][o] for BT batch rows.  Input channels go in
// batches of kMixIC: all W and X loads of a batch are issued (clamped
// indices, no branches) before any of its products, so each thread keeps
// about 8 (BT + 1) loads in flight; W, the largest operand when the channel
// counts are small, is read exactly once.
template <int BT>
__global__ __launch_bounds__(kThreads) void k_mix_valu(const float2* __restrict__ xh, MixAddr ax,
                                                      const float2* __restrict__ w, float2* __restrict__ yh,
                                                      MixAddr ay, int64_t B, int64_t Cin, int64_t Cout, int64_t M,
                                                      int ot_log2, int64_t n_ot, int64_t n_mt) {
    const int tid = threadIdx.x;
    const int64_t bid = blockIdx.x;
    const int64_t bx = bid % n_ot;
    const int64_t by = (bid / n_ot) % n_mt;
    const int64_t bz = bid / (n_ot * n_mt);
    const int64_t o = bx * (1 << ot_log2) + (tid & ((1 << ot_log2) - 1));
    const int64_t m = by * (kThreads >> ot_log2) + (tid >> ot_log2);
    const int64_t b0 = bz * BT;
    if (o >= Cout || m >= M) return;
    float2 acc[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[t] = make_float2(0.0f, 0.0f);
    for (int64_t i0 = 0; i0 < Cin; i0 += kMixIC) {
        float2 wv[kMixIC], xv[BT][kMixIC];
#pragma unroll
        for (int j = 0; j < kMixIC; ++j) {
            const int64_t i = i0 + j < Cin ? i0 + j : Cin - 1;
            wv[j] = w[(m * Cin + i) * Cout + o];
#pragma unroll
            for (int t = 0; t < BT; ++t) {
                const int64_t b = b0 + t < B ? b0 + t : B - 1;
                xv[t][j] = xh[ax.at(b, i, m)];
            }
        }
        // channels past Cin contribute nothing
#pragma unroll
        for (int j = 0; j < kMixIC; ++j)
            if (i0 + j >= Cin) wv[j] = make_float2(0.0f, 0.0f);
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int j = 0; j < kMixIC; ++j) acc[t] = cfma(acc[t], xv[t][j], wv[j]);
    }
#pragma unroll
    for (int t = 0; t < BT; ++t) {
        if (b0 + t < B) yh[ay.at(b0 + t, o, m)] = acc[t];
    }
}

#define FNO_LOG2_CASES(MACRO) \
    MACRO(1) MACRO(2) MACRO(3) MACRO(4) MACRO(5) MACRO(6) MACRO(7) MACRO(8) MACRO(9) MACRO(10) MACRO(11) MACRO(12)

int rows_per_block(int log2n) { return (1 << log2n) >= kLdsElems ? 1 : kLdsElems >> log2n; }

}  // namespace

hipError_t launch_rows_fwd(const float* x, float2* y, int64_t nrows, int log2W, int my, int y_ld, float scale,
                           const float2* tw, hipStream_t s) {
    if (rows_pruned_supported(log2W, my)) return launch_rows_fwd_pruned(x, y, nrows, log2W, my, y_ld, scale, tw, s);
    const int64_t npairs = (nrows + 1) / 2;
    const int p = rows_per_block(log2W);
    const dim3 grid((unsigned)((npairs + p - 1) / p));
    switch (log2W) {
#define CASE(L) \
    case L: return launch_kernel(k_rows_fwd<L>, grid, dim3(kThreads), 0, s, x, y, nrows, my, y_ld, scale, tw);
        FNO_LOG2_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rows_inv(const float2* y, float* out, int64_t nrows, int log2W, int my, int y_ld, float scale,
                           const float2* tw, hipStream_t s, const Epilogue& epi) {
    if (rows_pruned_supported(log2W, my))
        return launch_rows_inv_pruned(y, out, nrows, log2W, my, y_ld, scale, tw, s, epi);
    const int64_t npairs = (nrows + 1) / 2;
    const int p = rows_per_block(log2W);
    const dim3 grid((unsigned)((npairs + p - 1) / p));
    switch (log2W) {
#define CASE(L)                                                                                                   \
    case L:                                                                                                       \
        return epi.on ? launch_kernel(k_rows_inv<L, true>, grid, dim3(kThreads), 0, s, y, out, nrows, my, y_ld,   \
                                      scale, tw, epi)                                                             \
                      : launch_kernel(k_rows_inv<L, false>, grid, dim3(kThreads), 0, s, y, out, nrows, my, y_ld,  \
                                      scale, tw, epi);
        FNO_LOG2_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
}

static int cols_per_block(int log2H, int my) {
    const int cap = kLdsElems >> log2H;
    return cap < my ? cap : my;
}

hipError_t launch_cols_fwd(const float2* r, float2* xh, int64_t nimg, int log2H, int mx, int my, float scale,
                           const float2* tw, hipStream_t s) {
    if (cols_pruned_supported(log2H, mx, my)) return launch_cols_fwd_pruned(r, xh, nimg, log2H, mx, my, scale, tw, s);
    const int kb = cols_per_block(log2H, my);
    const int nkb = (my + kb - 1) / kb;
    const dim3 grid((unsigned)(nkb * nimg));
    switch (log2H) {
#define CASE(L) \
    case L: return launch_kernel(k_cols_fwd<L>, grid, dim3(kThreads), 0, s, r, xh, mx, my, kb, nkb, scale, tw);
        FNO_LOG2_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cols_inv(const float2* yh, float2* r, int64_t nimg, int log2H, int mx, int my,
                           const float2* tw, hipStream_t s) {
    if (cols_pruned_supported(log2H, mx, my)) return launch_cols_inv_pruned(yh, r, nimg, log2H, mx, my, tw, s);
    const int kb = cols_per_block(log2H, my);
    const int nkb = (my + kb - 1) / kb;
    const dim3 grid((unsigned)(nkb * nimg));
    switch (log2H) {
#define CASE(L) \
    case L: return launch_kernel(k_cols_inv<L>, grid, dim3(kThreads), 0, s, yh, r, mx, my, kb, nkb, tw);
        FNO_LOG2_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mix_valu(const float2* xh, const SpecLayout& lx, const float2* w, float2* yh,
                           const SpecLayout& ly, int64_t B, int64_t Cin, int64_t Cout, int64_t M, hipStream_t s) {
    int ot_log2 = 0;
    while ((1 << ot_log2) < Cout && ot_log2 < 6) ++ot_log2;
    const int64_t ot = 1 << ot_log2;
    const int64_t mt = kThreads >> ot_log2;
    const int64_t n_ot = (Cout + ot - 1) / ot;
    const int64_t n_mt = (M + mt - 1) / mt;
    // batch rows per thread: the fewest of 2, 4, 8 that cover B (8 past it)
    const int bt = B <= 2 ? 2 : (B <= 4 ? 4 : 8);
    const int64_t n_bt = (B + bt - 1) / bt;
    const int64_t nb = n_ot * n_mt * n_bt;
    if (nb >= INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nb);
    const MixAddr ax{lx.sb, lx.sc, lx.st};
    const MixAddr ay{ly.sb, ly.sc, ly.st};
    switch (bt) {
        case 2:
            return launch_kernel(k_mix_valu<2>, grid, dim3(kThreads), 0, s, xh, ax, w, yh, ay, B, Cin, Cout, M, ot_log2,
                                 n_ot, n_mt);
        case 4:
            return launch_kernel(k_mix_valu<4>, grid, dim3(kThreads), 0, s, xh, ax, w, yh, ay, B, Cin, Cout, M, ot_log2,
                                 n_ot, n_mt);
        default:
            return launch_kernel(k_mix_valu<8>, grid, dim3(kThreads), 0, s, xh, ax, w, yh, ay, B, Cin, Cout, M, ot_log2,
                                 n_ot, n_mt);
    }
}

}  // namespace fno
