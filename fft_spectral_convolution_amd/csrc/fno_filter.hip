// Diagonal global filter: the channel mix replaced by one complex weight
// per kept mode and channel (the learnable frequency mask of the TurboFNO
// blog, section 5.2, and the frequency-domain token mixing of the FFT blog,
// section 3.2):
//   yh(b, c, m) = xh(b, c, m) * mask[m][c].
// Pure streaming: two spectra and the (small, cache-resident) mask.  Both
// spectra share one layout; threads walk the layout's storage order, so
// reads and writes are contiguous.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kDiagThreads = 256;

// tiled: storage [b][m / 8][c][m % 8]; else canonical [b][c][m] with an even
// M.  e indexes complex pairs (elements 2e and 2e + 1: the same (b, c) and
// modes m, m + 1, which both layouts keep adjacent).
template <bool TILED>
__global__ __launch_bounds__(kDiagThreads) void k_mix_diag_pairs(const float2* __restrict__ xh, float2* __restrict__ yh,
                                                           const float2* __restrict__ mask, int64_t npairs, int C,
                                                           int M, int nt) {
    const int64_t stride = (int64_t)gridDim.x * kDiagThreads;
    for (int64_t e = (int64_t)blockIdx.x * kDiagThreads + threadIdx.x; e < npairs; e += stride) {
        const int64_t e2 = 2 * e;
        int c, m;
        if constexpr (TILED) {
            const int j = (int)(e2 & 7);
            const int64_t q = e2 >> 3;                       // (b, mt, c) run index
            c = (int)(q % C);
            m = 8 * (int)((q / C) % nt) + j;
        } else {
            m = (int)(e2 % M);
            c = (int)((e2 / M) % C);
        }
        const float4 v = reinterpret_cast<const float4*>(xh)[e];
        // modes past M (the tiled layout's padding) are written as zero
        const float2 y0 = m < M ? cmul(make_float2(v.x, v.y), mask[(int64_t)m * C + c]) : make_float2(0.0f, 0.0f);
        const float2 y1 =
            m + 1 < M ? cmul(make_float2(v.z, v.w), mask[(int64_t)(m + 1) * C + c]) : make_float2(0.0f, 0.0f);
        reinterpret_cast<float4*>(yh)[e] = make_float4(y0.x, y0.y, y1.x, y1.y);
    }
}

// canonical layout with an odd M: one complex element per thread
__global__ __launch_bounds__(kDiagThreads) void k_mix_diag_single(const float2* __restrict__ xh,
                                                                  float2* __restrict__ yh,
                                                                  const float2* __restrict__ mask, int64_t n, int C,
                                                                  int M) {
    const int64_t stride = (int64_t)gridDim.x * kDiagThreads;
    for (int64_t e = (int64_t)blockIdx.x * kDiagThreads + threadIdx.x; e < n; e += stride) {
        const int m = (int)(e % M);
        const int c = (int)((e / M) % C);
        yh[e] = cmul(xh[e], mask[(int64_t)m * C + c]);
    }
}

// mt[c][m] = mask[m][c]: 32 x 32 tiles through LDS
constexpr int kTrTile = 32;
__global__ __launch_bounds__(kDiagThreads) void k_mask_transpose(const float2* __restrict__ mask,
                                                                 float2* __restrict__ mt, int M, int C, int n_mt) {
    __shared__ float2 tile[kTrTile][kTrTile + 1];
    const int m0 = (int)(blockIdx.x % n_mt) * kTrTile;
    const int c0 = (int)(blockIdx.x / n_mt) * kTrTile;
    const int tx = threadIdx.x & (kTrTile - 1);
    const int ty = threadIdx.x / kTrTile;
    for (int r = ty; r < kTrTile; r += kDiagThreads / kTrTile)
        if (m0 + r < M && c0 + tx < C) tile[r][tx] = mask[(int64_t)(m0 + r) * C + c0 + tx];
    __syncthreads();
    for (int r = ty; r < kTrTile; r += kDiagThreads / kTrTile)
        if (c0 + r < C && m0 + tx < M) mt[(int64_t)(c0 + r) * M + m0 + tx] = tile[tx][r];
}

}  // namespace

hipError_t launch_mask_transpose(const float2* mask, float2* mt, int64_t M, int64_t C, hipStream_t s) {
    const int64_t n_mt = (M + kTrTile - 1) / kTrTile;
    const int64_t n = n_mt * ((C + kTrTile - 1) / kTrTile);
    if (n >= INT32_MAX || M > INT32_MAX || C > INT32_MAX) return hipErrorInvalidValue;
    return launch_kernel(k_mask_transpose, dim3((unsigned)n), dim3(kDiagThreads), 0, s, mask, mt, (int)M, (int)C,
                         (int)n_mt);
}

bool mix_diag_supported(const SpecLayout& lay, int64_t M) {
    return lay.sc == 8 ? lay.st == 8 * (int64_t)lay.C : (lay.sc == M && lay.st == 8);
}

hipError_t launch_mix_diag(const float2* xh, float2* yh, const SpecLayout& lay, const float2* mask, int64_t B,
                           int64_t C, int64_t M, hipStream_t s) {
    if (!mix_diag_supported(lay, M) || C > INT32_MAX || M > INT32_MAX) return hipErrorInvalidValue;
    const bool tiled = lay.sc == 8;
    const int64_t nt = (M + 7) / 8;
    const int64_t elems = tiled ? B * nt * C * 8 : B * C * M;   // complex elements in storage
    const bool pairs = tiled || M % 2 == 0;
    const int64_t items = pairs ? elems / 2 : elems;
    int64_t blocks = (items + kDiagThreads - 1) / kDiagThreads;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    const dim3 grid((unsigned)blocks);
    if (!pairs)
        return launch_kernel(k_mix_diag_single, grid, dim3(kDiagThreads), 0, s, xh, yh, mask, items, (int)C, (int)M);
    if (tiled)
        return launch_kernel(k_mix_diag_pairs<true>, grid, dim3(kDiagThreads), 0, s, xh, yh, mask, items, (int)C,
                             (int)M, (int)nt);
    return launch_kernel(k_mix_diag_pairs<false>, grid, dim3(kDiagThreads), 0, s, xh, yh, mask, items, (int)C,
                         (int)M, (int)nt);
}

}  // namespace fno
