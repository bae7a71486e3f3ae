// Per-mode channel mix on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).
//
// For every kept mode m the mix is a complex GEMM (TurboFNO blog, section 2.2:
// the frequency-domain GEMM is a per-mode complex multiply-accumulate,
// (a+bi)(c+di) = (ac-bd) + (ad+bc)i):
//   Y_m[b][o] = sum_i X_m[b][i] * W_m[i][o]
// done as four real products, Yr += Xr Wr - Xi Wi and Yi += Xr Wi + Xi Wr,
// all accumulated in fp32.
//
// Workgroup = 8 waves = one tile of 8 consecutive modes x 32 batch rows x 64
// output channels; wave w owns mode m0 + w (a 32x64 complex accumulator =
// four 32x32 fp32 MFMA blocks).  The input channels are consumed in chunks of
// 8: the X chunk of all 8 modes ([32 b][8 i][8 m], one 64-byte run per
// (b, i)) is staged in LDS and shared by the 8 waves; each wave streams its
// own W_m rows straight from global memory into the B operand, one chunk ahead.
// The result goes back through LDS so every (b, o) writes its 8 modes as one
// 64-byte run.  Rows, channels and modes past the ends are masked.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMixWaves = 8;           // = modes per tile
constexpr int kMixThreads = 64 * kMixWaves;
constexpr int kMixKC = 8;              // input channels per chunk
constexpr int kMixBRows = 32;          // batch rows per tile (MFMA M)
constexpr int kMixOCols = 64;          // output channels per tile (2 MFMA N blocks)

struct Addr {
    int64_t sb, sc, st;
    __device__ __forceinline__ int64_t at(int64_t b, int64_t c, int64_t m) const {
        return b * sb + c * sc + (m >> 3) * st + (m & 7);
    }
};

__device__ __forceinline__ floatx16 mfma32(float a, float b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kMixThreads) void k_mix_mfma(const float2* __restrict__ xh, Addr ax,
                                                          const float2* __restrict__ w, float2* __restrict__ yh,
                                                          Addr ay, int B, int Cin, int Cout, int M, int n_mt,
                                                          int n_bt) {
    __shared__ float2 a_lds[kMixBRows * kMixKC * 8];      // [b][i][m] chunk, 16 KiB
    __shared__ float2 y_lds[8 * kMixOCols * 8];           // [b8][o][m] output staging, 32 KiB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int mt = blockIdx.x % n_mt;
    const int bt = (blockIdx.x / n_mt) % n_bt;
    const int ot = blockIdx.x / (n_mt * n_bt);
    const int m0 = mt * 8;
    const int b0 = bt * kMixBRows;
    const int o0 = ot * kMixOCols;
    const int m = m0 + wave;                 // this wave's mode
    const bool m_ok = m < M;
    const int lrow = lane & 31;              // MFMA row (A) / column (B, C)
    const int lk = lane >> 5;                // MFMA k index within a step

    floatx16 cr0 = {}, cr1 = {}, ci0 = {}, ci1 = {};

    // W operand for input channel i, output channels o0 + nb*32 + lrow
    auto load_w = [&](int ic, float2 (&wv)[8]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int i = ic + 2 * s + lk;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int o = o0 + nb * 32 + lrow;
                float2 v = make_float2(0.0f, 0.0f);
                if (m_ok && i < Cin && o < Cout) v = w[((int64_t)m * Cin + i) * Cout + o];
                wv[s * 2 + nb] = v;
            }
        }
    };

    float2 wcur[8], wnext[8];
    load_w(0, wcur);

    for (int ic = 0; ic < Cin; ic += kMixKC) {
        // stage X[b0:b0+32][ic:ic+8][m0:m0+8]: thread -> (b, i, half of the 8 modes)
        {
            const int e = tid;                       // 512 items = 32 b x 8 i x 2 halves
            const int bl = e >> 4;
            const int il = (e >> 1) & 7;
            const int half = e & 1;
            const int b = b0 + bl;
            const int i = ic + il;
            float2 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int mm = m0 + half * 4 + q;
                v[q] = (b < B && i < Cin && mm < M) ? xh[ax.at(b, i, mm)] : make_float2(0.0f, 0.0f);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) a_lds[(bl * kMixKC + il) * 8 + half * 4 + q] = v[q];
        }
        if (ic + kMixKC < Cin) load_w(ic + kMixKC, wnext);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float2 a = a_lds[(lrow * kMixKC + 2 * s + lk) * 8 + wave];
            const float2 w0 = wcur[s * 2 + 0];
            const float2 w1 = wcur[s * 2 + 1];
            cr0 = mfma32(a.x, w0.x, cr0);
            cr0 = mfma32(-a.y, w0.y, cr0);
            ci0 = mfma32(a.x, w0.y, ci0);
            ci0 = mfma32(a.y, w0.x, ci0);
            cr1 = mfma32(a.x, w1.x, cr1);
            cr1 = mfma32(-a.y, w1.y, cr1);
            ci1 = mfma32(a.x, w1.y, ci1);
            ci1 = mfma32(a.y, w1.x, ci1);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) wcur[q] = wnext[q];
    }

    // C layout of the 32x32 block: lane holds column lrow and, in register r,
    // row 8 * (r / 4) + 4 * lk + (r % 4).
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {              // 8 batch rows per round
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rr * 4 + q;
            const int bl = 4 * lk + q;               // row within the round
            y_lds[(bl * kMixOCols + lrow) * 8 + wave] = make_float2(cr0[r], ci0[r]);
            y_lds[(bl * kMixOCols + 32 + lrow) * 8 + wave] = make_float2(cr1[r], ci1[r]);
        }
        __syncthreads();
        {
            const int e = tid;                       // 512 items = 8 b x 64 o
            const int bl = e >> 6;
            const int ol = e & 63;
            const int b = b0 + rr * 8 + bl;
            const int o = o0 + ol;
            if (b < B && o < Cout) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int mm = m0 + q;
                    if (mm < M) yh[ay.at(b, o, mm)] = y_lds[(bl * kMixOCols + ol) * 8 + q];
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_mix_mfma(const float2* xh, const SpecLayout& lx, const float2* w, float2* yh, const SpecLayout& ly,
                           int64_t B, int64_t Cin, int64_t Cout, int64_t M, hipStream_t s) {
    const int n_mt = (int)((M + 7) / 8);
    const int n_bt = (int)((B + kMixBRows - 1) / kMixBRows);
    const int n_ot = (int)((Cout + kMixOCols - 1) / kMixOCols);
    const Addr ax{lx.sb, lx.sc, lx.st};
    const Addr ay{ly.sb, ly.sc, ly.st};
    const dim3 grid((unsigned)((int64_t)n_mt * n_bt * n_ot));
    hipLaunchKernelGGL(k_mix_mfma, grid, dim3(kMixThreads), 0, s, xh, ax, w, yh, ay, (int)B, (int)Cin, (int)Cout,
                       (int)M, n_mt, n_bt);
    return hipGetLastError();
}

}  // namespace fno
