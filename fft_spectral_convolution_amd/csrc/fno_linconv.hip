// Helpers of the zero-padded linear convolution (the FFT blog, sections
// 2.1 and 5.1-5.2: pad input and kernel, R2C, pointwise product, C2R,
// crop).  The transforms and the per-frequency channel product are the
// spectral convolution's own kernels at full modes (the row kernels pad the
// input and crop the output themselves); this file adds the zero-padding
// copy of the kernels and the weight spectrum's layout change.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kLcThreads = 256;
constexpr int kLcTile = 32;

int64_t grid_for(int64_t n) {
    int64_t b = (n + kLcThreads - 1) / kLcThreads;
    return b < 1 ? 1 : (b > 65536 ? 65536 : b);
}

// dst[img][p][q] = src[img][p][q] for p < H, q < W, else 0 (dst PH x PW)
__global__ __launch_bounds__(kLcThreads) void k_pad2d(const float* __restrict__ src, float* __restrict__ dst,
                                                      int64_t n, int H, int W, int PH, int PW) {
    const int64_t stride = (int64_t)gridDim.x * kLcThreads;
    for (int64_t e = (int64_t)blockIdx.x * kLcThreads + threadIdx.x; e < n; e += stride) {
        const int q = (int)(e % PW);
        const int64_t r = e / PW;
        const int p = (int)(r % PH);
        const int64_t img = r / PH;
        dst[e] = (p < H && q < W) ? src[(img * H + p) * W + q] : 0.0f;
    }
}

// w[m][i][o] = scale * kh[o * Cin + i][m]: a 32 x 32 tile of (m, i Cout + o)
// per workgroup, read along m and written along (i, o) through LDS
__global__ __launch_bounds__(kLcThreads) void k_spec_to_weight(const float2* __restrict__ kh, float2* __restrict__ w,
                                                               int64_t M, int Cin, int Cout, float scale,
                                                               int64_t n_mt, int64_t n_ct) {
    __shared__ float2 tile[kLcTile][kLcTile + 1];
    const int64_t mt = blockIdx.x % n_mt;
    const int64_t ct = blockIdx.x / n_mt;
    const int tx = threadIdx.x & (kLcTile - 1);
    const int ty = threadIdx.x / kLcTile;
    const int64_t IO = (int64_t)Cin * Cout;
    for (int r = ty; r < kLcTile; r += kLcThreads / kLcTile) {
        const int64_t c = ct * kLcTile + r;                 // c = i Cout + o
        const int64_t m = mt * kLcTile + tx;
        if (c < IO && m < M) {
            const int64_t i = c / Cout, o = c % Cout;
            tile[r][tx] = kh[(o * Cin + i) * M + m];
        }
    }
    __syncthreads();
    for (int r = ty; r < kLcTile; r += kLcThreads / kLcTile) {
        const int64_t m = mt * kLcTile + r;
        const int64_t c = ct * kLcTile + tx;
        if (c < IO && m < M) w[m * IO + c] = cscale(tile[tx][r], scale);
    }
}

}  // namespace

hipError_t launch_pad2d(const float* src, float* dst, int64_t nimg, int H, int W, int PH, int PW, hipStream_t s) {
    const int64_t n = nimg * PH * PW;
    return launch_kernel(k_pad2d, dim3((unsigned)grid_for(n)), dim3(kLcThreads), 0, s, src, dst, n, H, W, PH, PW);
}

hipError_t launch_spec_to_weight(const float2* kh, float2* w, int64_t M, int64_t Cin, int64_t Cout, float scale,
                                 hipStream_t s) {
    const int64_t n_mt = (M + kLcTile - 1) / kLcTile;
    const int64_t n_ct = (Cin * Cout + kLcTile - 1) / kLcTile;
    if (n_mt * n_ct >= INT32_MAX || Cin > INT32_MAX || Cout > INT32_MAX) return hipErrorInvalidValue;
    return launch_kernel(k_spec_to_weight, dim3((unsigned)(n_mt * n_ct)), dim3(kLcThreads), 0, s, kh, w, M, (int)Cin,
                         (int)Cout, scale, n_mt, n_ct);
}

}  // namespace fno
