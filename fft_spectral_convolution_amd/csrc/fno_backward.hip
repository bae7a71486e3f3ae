// Kernels of the backward pass: gradients of a real loss L through the
// spectral convolution, given g = dL/dout.
//
// With the kept modes m, X = the truncated forward transform of x, G the one
// of g and c_m the complex-to-real weight of the mode's ky (1 for ky = 0 and
// ky = W/2, 2 otherwise; FFT blog, section 2.2: C2R from the N/2+1 half
// spectrum), the chain rule through the per-mode product Y = X W (TurboFNO
// blog, section 2.2) gives
//   dL/dx = the same forward -> mix -> inverse chain applied to g with the
//           conjugate-transposed weight W^H[m][o][i] = conj W[m][i][o]
//           (the C2R weights of the inverse already account for c_m);
//   dL/dRe W + i dL/dIm W = c_m sum_b conj(X[b][i][m]) G[b][o][m].
// The transforms and the mix are the forward pass's kernels; this file adds
// the weight adjoint (a conjugating transpose per mode) and the weight
// gradient (a per-mode contraction over the batch).
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kAdjTile = 32;
constexpr int kAdjThreads = 256;
constexpr int kGradThreads = 256;
constexpr int kGradKB = 8;       // batch items per batch of loads

// (b, c, m) -> complex element offset of a truncated spectrum
struct SpecAddr {
    int64_t sb, sc, st;
    __device__ __forceinline__ int64_t at(int64_t b, int64_t c, int64_t m) const {
        return b * sb + c * sc + (m >> 3) * st + (m & 7);
    }
};

// wt[m][o][i] = conj(w[m][i][o]): workgroup (m, tile) moves a 32 x 32 tile of
// one mode, read along o and written along i through LDS.
__global__ __launch_bounds__(kAdjThreads) void k_weight_adjoint(const float2* __restrict__ w, float2* __restrict__ wt,
                                                                int Cin, int Cout, int n_ti, int n_to) {
    __shared__ float2 tile[kAdjTile][kAdjTile + 1];
    const int64_t tiles = (int64_t)n_ti * n_to;
    const int64_t m = blockIdx.x / tiles;
    const int t = (int)(blockIdx.x % tiles);
    const int i0 = (t / n_to) * kAdjTile;
    const int o0 = (t % n_to) * kAdjTile;
    const int tx = threadIdx.x & (kAdjTile - 1);
    const int ty = threadIdx.x / kAdjTile;
    const float2* src = w + m * (int64_t)Cin * Cout;
    for (int r = ty; r < kAdjTile; r += kAdjThreads / kAdjTile) {
        const int i = i0 + r, o = o0 + tx;
        if (i < Cin && o < Cout) tile[r][tx] = src[(int64_t)i * Cout + o];
    }
    __syncthreads();
    float2* dst = wt + m * (int64_t)Cin * Cout;
    for (int r = ty; r < kAdjTile; r += kAdjThreads / kAdjTile) {
        const int o = o0 + r, i = i0 + tx;
        if (i < Cin && o < Cout) {
            const float2 v = tile[tx][r];
            dst[(int64_t)o * Cin + i] = make_float2(v.x, -v.y);
        }
    }
}

// gw[m][i][o] = c_m sum_b conj(xh(b, i, m)) gh(b, o, m).  Thread (m, o)
// accumulates BT input channels; the batch is walked kGradKB items at a
// time, all loads of a batch issued (clamped indices, no branches) before
// any product.
template <int BT>
__global__ __launch_bounds__(kGradThreads) void k_weight_grad(const float2* __restrict__ xh, SpecAddr ax,
                                                              const float2* __restrict__ gh, SpecAddr ag,
                                                              float2* __restrict__ gw, int64_t B, int64_t Cin,
                                                              int64_t Cout, int64_t M, int my, int nyq, int ot_log2,
                                                              int64_t n_ot, int64_t n_mt) {
    const int tid = threadIdx.x;
    const int64_t bid = blockIdx.x;
    const int64_t bx = bid % n_ot;
    const int64_t by = (bid / n_ot) % n_mt;
    const int64_t bz = bid / (n_ot * n_mt);
    const int64_t o = bx * (1 << ot_log2) + (tid & ((1 << ot_log2) - 1));
    const int64_t m = by * (kGradThreads >> ot_log2) + (tid >> ot_log2);
    const int64_t i0 = bz * BT;
    if (o >= Cout || m >= M) return;
    float2 acc[BT];
#pragma unroll
    for (int t = 0; t < BT; ++t) acc[t] = make_float2(0.0f, 0.0f);
    for (int64_t b0 = 0; b0 < B; b0 += kGradKB) {
        float2 gv[kGradKB], xv[BT][kGradKB];
#pragma unroll
        for (int j = 0; j < kGradKB; ++j) {
            const int64_t b = b0 + j < B ? b0 + j : B - 1;
            gv[j] = gh[ag.at(b, o, m)];
#pragma unroll
            for (int t = 0; t < BT; ++t) {
                const int64_t i = i0 + t < Cin ? i0 + t : Cin - 1;
                xv[t][j] = xh[ax.at(b, i, m)];
            }
        }
        // batch items past B contribute nothing
#pragma unroll
        for (int j = 0; j < kGradKB; ++j)
            if (b0 + j >= B) gv[j] = make_float2(0.0f, 0.0f);
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int j = 0; j < kGradKB; ++j) {
                // conj(x) g = (x.x g.x + x.y g.y) + i (x.x g.y - x.y g.x)
                const float2 xx = xv[t][j], g = gv[j];
                acc[t].x = fmaf(xx.x, g.x, acc[t].x);
                acc[t].x = fmaf(xx.y, g.y, acc[t].x);
                acc[t].y = fmaf(xx.x, g.y, acc[t].y);
                acc[t].y = fmaf(-xx.y, g.x, acc[t].y);
            }
    }
    const int ky = (int)(m % my);
    const float c = (ky == 0 || ky == nyq) ? 1.0f : 2.0f;
#pragma unroll
    for (int t = 0; t < BT; ++t)
        if (i0 + t < Cin) gw[(m * Cin + i0 + t) * Cout + o] = cscale(acc[t], c);
}

}  // namespace

hipError_t launch_weight_adjoint(const float2* w, float2* wt, int64_t M, int64_t Cin, int64_t Cout, hipStream_t s) {
    const int64_t n_ti = (Cin + kAdjTile - 1) / kAdjTile;
    const int64_t n_to = (Cout + kAdjTile - 1) / kAdjTile;
    const int64_t nb = M * n_ti * n_to;
    if (nb >= INT32_MAX || Cin > INT32_MAX || Cout > INT32_MAX) return hipErrorInvalidValue;
    return launch_kernel(k_weight_adjoint, dim3((unsigned)nb), dim3(kAdjThreads), 0, s, w, wt, (int)Cin, (int)Cout,
                         (int)n_ti, (int)n_to);
}

hipError_t launch_weight_grad(const float2* xh, const SpecLayout& lx, const float2* gh, const SpecLayout& lg,
                              float2* gw, int64_t B, int64_t Cin, int64_t Cout, int64_t M, int my, int nyq,
                              hipStream_t s) {
    int ot_log2 = 0;
    while ((1 << ot_log2) < Cout && ot_log2 < 6) ++ot_log2;
    const int64_t n_ot = (Cout + (1 << ot_log2) - 1) >> ot_log2;
    const int64_t mt = kGradThreads >> ot_log2;
    const int64_t n_mt = (M + mt - 1) / mt;
    // input channels per thread: the fewest of 2, 4, 8 that cover Cin (8 past it)
    const int bt = Cin <= 2 ? 2 : (Cin <= 4 ? 4 : 8);
    const int64_t n_it = (Cin + bt - 1) / bt;
    const int64_t nb = n_ot * n_mt * n_it;
    if (nb >= INT32_MAX) return hipErrorInvalidValue;
    const SpecAddr ax{lx.sb, lx.sc, lx.st};
    const SpecAddr ag{lg.sb, lg.sc, lg.st};
    const dim3 grid((unsigned)nb);
    switch (bt) {
        case 2:
            return launch_kernel(k_weight_grad<2>, grid, dim3(kGradThreads), 0, s, xh, ax, gh, ag, gw, B, Cin, Cout, M,
                                 my, nyq, ot_log2, n_ot, n_mt);
        case 4:
            return launch_kernel(k_weight_grad<4>, grid, dim3(kGradThreads), 0, s, xh, ax, gh, ag, gw, B, Cin, Cout, M,
                                 my, nyq, ot_log2, n_ot, n_mt);
        default:
            return launch_kernel(k_weight_grad<8>, grid, dim3(kGradThreads), 0, s, xh, ax, gh, ag, gw, B, Cin, Cout, M,
                                 my, nyq, ot_log2, n_ot, n_mt);
    }
}

}  // namespace fno
