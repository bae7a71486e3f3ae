// Fused per-image forward and inverse transforms for grids with H, W <= 128.
//
// Forward (one workgroup per image): the real rows are transformed two at a
// time as one complex row z = x[p] + i x[p + H/2]; only the bins a truncated
// row spectrum needs (ky < my and their mirrors W - ky) are kept in LDS.
// The column pass then rebuilds each row's half spectrum on the fly
// (A = (Z[k] + conj Z[-k]) / 2, B = (Z[k] - conj Z[-k]) / 2i), transforms the
// my columns along H and writes only kx in [0,mx) u [H-mx,H), scaled.
// Inverse: the mirror image -- zero-filled columns are inverted straight from
// the truncated spectrum into LDS, then pairs of rows are turned back into
// real rows by one complex inverse transform of Ya + i Yb (Hermitian
// extensions, imaginary parts of the DC / Nyquist bins dropped).  (TurboFNO
// blog sections 2.1-2.2: row and column transforms in one kernel with the
// intermediate in on-chip memory; FFT blog section 2.2: R2C / C2R half
// spectra.)
//
// Each length-N transform is split N = R1 * R2: a thread holds R1 points
// (n = t + R2 m), does an R1-point DFT in registers, multiplies by
// W_N^{t k1} and hands the R1 results through LDS to the R2 threads that do
// the R2-point DFTs across t, giving X[k1 + R1 k2].
//
// Spectra outside the kernels use a mode-addressed layout:
//   addr(b, c, m) = b * sb + c * sc + (m / 8) * st + (m % 8)   [complex elements]
// with m = (s * mx + r) * my + ky the weight's mode order.  The canonical
// layout [B][C][M] is sb = C*M, sc = M, st = 8; the tiled layout used between
// the fused kernels, [B][M/8][C][8], is sb = (M/8)*C*8, sc = 8, st = C*8 --
// every 8 consecutive modes of one (b, c) are one 64-byte chunk.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kSmallThreads = 256;

template <int N> struct Split;
template <> struct Split<8>   { static constexpr int R1 = 4,  R2 = 2; };
template <> struct Split<16>  { static constexpr int R1 = 4,  R2 = 4; };
template <> struct Split<32>  { static constexpr int R1 = 8,  R2 = 4; };
template <> struct Split<64>  { static constexpr int R1 = 8,  R2 = 8; };
template <> struct Split<128> { static constexpr int R1 = 16, R2 = 8; };

__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }

struct ModeAddr {
    int64_t sb, sc, st;
    int C;
    __device__ __forceinline__ int64_t at(int64_t img, int m) const {
        const int64_t b = img / C;
        const int64_t c = img - b * C;
        return b * sb + c * sc + (int64_t)(m >> 3) * st + (m & 7);
    }
};

template <int LOG2H, int LOG2W>
struct SmallPlan {
    static constexpr int H = 1 << LOG2H;
    static constexpr int W = 1 << LOG2W;
    static constexpr int P = H / 2;                 // complex rows (real row pairs)
    static constexpr int R1W = Split<W>::R1, R2W = Split<W>::R2;
    static constexpr int R1H = Split<H>::R1, R2H = Split<H>::R2;
    static constexpr int XSW = R1W + 1;             // padded per-thread slot (rows)
    static constexpr int XSH = R1H + 1;             // padded per-thread slot (cols)
    static constexpr int ROWS_IT = kSmallThreads / R2W;
    static constexpr int COLS_IT = kSmallThreads / R2H;
    static constexpr int XBUF = (ROWS_IT * R2W * XSW > COLS_IT * R2H * XSH) ? ROWS_IT * R2W * XSW
                                                                              : COLS_IT * R2H * XSH;
    static_assert(R1W >= R2W && R1W % R2W == 0, "row split");
    static_assert(R1H >= R2H && R1H % R2H == 0 && R1H >= 2, "column split");
    // LDS: twiddles for W and H, two spectrum planes of H/2 x my (forward) or
    // one plane of H x my (inverse), and the exchange buffer.
    static size_t lds_bytes(int my) { return sizeof(float2) * ((size_t)W + H + (size_t)H * my + XBUF); }
};

template <int LOG2H, int LOG2W>
__global__ __launch_bounds__(kSmallThreads) void k_fwd2d_small(const float* __restrict__ x, float2* __restrict__ xh,
                                                              ModeAddr ma, int mx, int my, float scale,
                                                              const float2* __restrict__ tw) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int H = S::H, W = S::W, P = S::P;
    constexpr int R1W = S::R1W, R2W = S::R2W, R1H = S::R1H, R2H = S::R2H;
    extern __shared__ float2 smem[];
    float2* twW = smem;
    float2* twH = twW + W;
    float2* zlo = twH + H;              // [P][my]: Z_p[k], k < my
    float2* zhi = zlo + P * my;         // [P][my]: Z_p[(W - k) mod W]
    float2* xbuf = zhi + P * my;

    const int tid = threadIdx.x;
    const int64_t img = blockIdx.x;
    for (int j = tid; j < W; j += kSmallThreads) twW[j] = tw[j * (kNMax / W)];
    for (int j = tid; j < H; j += kSmallThreads) twH[j] = tw[j * (kNMax / H)];
    __syncthreads();

    const float* xi = x + img * (int64_t)(H * W);

    // ---- rows: complex row p = x[p] + i x[p + P] --------------------------
    {
        const int pl = tid / R2W;
        const int t = tid % R2W;
        float2* xb = xbuf + pl * (R2W * S::XSW);
        for (int p0 = 0; p0 < P; p0 += S::ROWS_IT) {
            const int p = p0 + pl;
            const bool active = p < P;
            if (active) {
                const float* ra = xi + p * W;
                const float* rb = ra + P * W;
                float2 v[R1W];
#pragma unroll
                for (int m = 0; m < R1W; ++m) v[m] = make_float2(ra[t + R2W * m], rb[t + R2W * m]);
                dft<R1W, -1>(v);
#pragma unroll
                for (int k1 = 1; k1 < R1W; ++k1) v[k1] = cmul(v[k1], twW[(t * k1) & (W - 1)]);
#pragma unroll
                for (int k1 = 0; k1 < R1W; ++k1) xb[t * S::XSW + k1] = v[k1];
            }
            __syncthreads();
            if (active) {
                const int p = p0 + pl;
#pragma unroll
                for (int j = 0; j < R1W / R2W; ++j) {
                    const int k1 = t + R2W * j;
                    float2 u[R2W];
#pragma unroll
                    for (int tt = 0; tt < R2W; ++tt) u[tt] = xb[tt * S::XSW + k1];
                    dft<R2W, -1>(u);
#pragma unroll
                    for (int k2 = 0; k2 < R2W; ++k2) {
                        const int k = k1 + R1W * k2;
                        if (k < my) zlo[p * my + k] = u[k2];
                        const int km = (W - k) & (W - 1);
                        if (km < my) zhi[p * my + km] = u[k2];
                    }
                }
            }
            __syncthreads();
        }
    }

    // ---- columns ky < my along H, kept kx only ------------------------------
    {
        const int t = tid / S::COLS_IT;
        const int cl = tid % S::COLS_IT;
        float2* xb = xbuf + cl * (R2H * S::XSH);
        for (int c0 = 0; c0 < my; c0 += S::COLS_IT) {
            const int ky = c0 + cl;
            const bool active = ky < my;
            if (active) {
                float2 v[R1H];
#pragma unroll
                for (int m = 0; m < R1H / 2; ++m) {
                    const int p = t + R2H * m;
                    const float2 zl = zlo[p * my + ky];
                    const float2 zm = zhi[p * my + ky];
                    v[m] = make_float2(0.5f * (zl.x + zm.x), 0.5f * (zl.y - zm.y));
                    v[m + R1H / 2] = make_float2(0.5f * (zl.y + zm.y), -0.5f * (zl.x - zm.x));
                }
                dft<R1H, -1>(v);
#pragma unroll
                for (int k1 = 1; k1 < R1H; ++k1) v[k1] = cmul(v[k1], twH[(t * k1) & (H - 1)]);
#pragma unroll
                for (int k1 = 0; k1 < R1H; ++k1) xb[t * S::XSH + k1] = v[k1];
            }
            __syncthreads();
            if (active) {
#pragma unroll
                for (int j = 0; j < R1H / R2H; ++j) {
                    const int k1 = t + R2H * j;
                    float2 u[R2H];
#pragma unroll
                    for (int tt = 0; tt < R2H; ++tt) u[tt] = xb[tt * S::XSH + k1];
                    dft<R2H, -1>(u);
#pragma unroll
                    for (int k2 = 0; k2 < R2H; ++k2) {
                        const int kx = k1 + R1H * k2;
                        const int q = kx < mx ? kx : (kx >= H - mx ? kx - H + 2 * mx : -1);
                        if (q >= 0) xh[ma.at(img, q * my + ky)] = cscale(u[k2], scale);
                    }
                }
            }
            __syncthreads();
        }
    }
}

template <int LOG2H, int LOG2W>
__global__ __launch_bounds__(kSmallThreads) void k_inv2d_small(const float2* __restrict__ yh, float* __restrict__ out,
                                                              ModeAddr ma, int mx, int my, float scale,
                                                              const float2* __restrict__ tw) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int H = S::H, W = S::W, P = S::P;
    constexpr int R1W = S::R1W, R2W = S::R2W, R1H = S::R1H, R2H = S::R2H;
    extern __shared__ float2 smem[];
    float2* twW = smem;
    float2* twH = twW + W;
    float2* rp = twH + H;               // [H][my]: column-inverted spectrum R'[h][ky]
    float2* xbuf = rp + H * my;

    const int tid = threadIdx.x;
    const int64_t img = blockIdx.x;
    for (int j = tid; j < W; j += kSmallThreads) twW[j] = tw[j * (kNMax / W)];
    for (int j = tid; j < H; j += kSmallThreads) twH[j] = tw[j * (kNMax / H)];
    __syncthreads();

    // ---- columns: R'[h][ky] = sum_{kept kx} Y[kx][ky] W_H^{+h kx} -------------
    {
        const int t = tid / S::COLS_IT;
        const int cl = tid % S::COLS_IT;
        float2* xb = xbuf + cl * (R2H * S::XSH);
        for (int c0 = 0; c0 < my; c0 += S::COLS_IT) {
            const int ky = c0 + cl;
            const bool active = ky < my;
            if (active) {
#pragma unroll
                for (int j = 0; j < R1H / R2H; ++j) {
                    const int k1 = t + R2H * j;
                    float2 u[R2H];
#pragma unroll
                    for (int k2 = 0; k2 < R2H; ++k2) {
                        const int kx = k1 + R1H * k2;
                        const int q = kx < mx ? kx : (kx >= H - mx ? kx - H + 2 * mx : -1);
                        u[k2] = q >= 0 ? yh[ma.at(img, q * my + ky)] : make_float2(0.0f, 0.0f);
                    }
                    dft<R2H, +1>(u);
#pragma unroll
                    for (int tt = 1; tt < R2H; ++tt) u[tt] = cmul(u[tt], conjf2(twH[(tt * k1) & (H - 1)]));
#pragma unroll
                    for (int tt = 0; tt < R2H; ++tt) xb[tt * S::XSH + k1] = u[tt];
                }
            }
            __syncthreads();
            if (active) {
                float2 v[R1H];
#pragma unroll
                for (int k1 = 0; k1 < R1H; ++k1) v[k1] = xb[t * S::XSH + k1];
                dft<R1H, +1>(v);
#pragma unroll
                for (int m = 0; m < R1H; ++m) rp[(t + R2H * m) * my + ky] = v[m];
            }
            __syncthreads();
        }
    }

    // ---- rows: two real rows per complex inverse transform -----------------
    {
        const int pl = tid / R2W;
        const int t = tid % R2W;
        float2* xb = xbuf + pl * (R2W * S::XSW);
        float* oi = out + img * (int64_t)(H * W);
        for (int p0 = 0; p0 < P; p0 += S::ROWS_IT) {
            const int p = p0 + pl;
            const bool active = p < P;
            if (active) {
                const float2* ya_row = rp + p * my;
                const float2* yb_row = rp + (p + P) * my;
#pragma unroll
                for (int j = 0; j < R1W / R2W; ++j) {
                    const int k1 = t + R2W * j;
                    float2 u[R2W];
#pragma unroll
                    for (int k2 = 0; k2 < R2W; ++k2) {
                        const int k = k1 + R1W * k2;
                        const int kk = k <= W / 2 ? k : W - k;
                        float2 z = make_float2(0.0f, 0.0f);
                        if (kk < my) {
                            const float2 ya = ya_row[kk];
                            const float2 yb = yb_row[kk];
                            if (kk == 0 || 2 * kk == W) z = make_float2(ya.x, yb.x);
                            else if (k == kk) z = make_float2(ya.x - yb.y, ya.y + yb.x);
                            else z = make_float2(ya.x + yb.y, yb.x - ya.y);
                        }
                        u[k2] = z;
                    }
                    dft<R2W, +1>(u);
#pragma unroll
                    for (int tt = 1; tt < R2W; ++tt) u[tt] = cmul(u[tt], conjf2(twW[(tt * k1) & (W - 1)]));
#pragma unroll
                    for (int tt = 0; tt < R2W; ++tt) xb[tt * S::XSW + k1] = u[tt];
                }
            }
            __syncthreads();
            if (active) {
                float2 v[R1W];
#pragma unroll
                for (int k1 = 0; k1 < R1W; ++k1) v[k1] = xb[t * S::XSW + k1];
                dft<R1W, +1>(v);
                float* oa = oi + p * W;
                float* ob = oa + P * W;
#pragma unroll
                for (int m = 0; m < R1W; ++m) {
                    oa[t + R2W * m] = v[m].x * scale;
                    ob[t + R2W * m] = v[m].y * scale;
                }
            }
            __syncthreads();
        }
    }
}

#define FNO_SMALL_CASES(MACRO) \
    MACRO(3, 3) MACRO(3, 4) MACRO(3, 5) MACRO(3, 6) MACRO(3, 7) \
    MACRO(4, 3) MACRO(4, 4) MACRO(4, 5) MACRO(4, 6) MACRO(4, 7) \
    MACRO(5, 3) MACRO(5, 4) MACRO(5, 5) MACRO(5, 6) MACRO(5, 7) \
    MACRO(6, 3) MACRO(6, 4) MACRO(6, 5) MACRO(6, 6) MACRO(6, 7) \
    MACRO(7, 3) MACRO(7, 4) MACRO(7, 5) MACRO(7, 6) MACRO(7, 7)

ModeAddr make_addr(const SpecLayout& l) {
    ModeAddr a;
    a.sb = l.sb;
    a.sc = l.sc;
    a.st = l.st;
    a.C = l.C;
    return a;
}

}  // namespace

bool small2d_supported(int log2H, int log2W, int my) {
    if (log2H < 3 || log2H > 7 || log2W < 3 || log2W > 7) return false;
    const size_t need = sizeof(float2) * ((size_t)(1 << log2W) + (1 << log2H) + (size_t)(1 << log2H) * my + 256 * 17);
    return need <= 150 * 1024;
}

hipError_t launch_fwd2d_small(const float* x, float2* xh, const SpecLayout& lay, int64_t nimg, int log2H, int log2W,
                              int mx, int my, float scale, const float2* tw, hipStream_t s) {
    const ModeAddr ma = make_addr(lay);
    switch (log2H * 16 + log2W) {
#define CASE(LH, LW)                                                                                          \
    case LH * 16 + LW: {                                                                                      \
        const size_t lds = SmallPlan<LH, LW>::lds_bytes(my);                                                  \
        hipLaunchKernelGGL((k_fwd2d_small<LH, LW>), dim3((unsigned)nimg), dim3(kSmallThreads), lds, s, x, xh, \
                           ma, mx, my, scale, tw);                                                            \
        break;                                                                                                \
    }
        FNO_SMALL_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_inv2d_small(const float2* yh, float* out, const SpecLayout& lay, int64_t nimg, int log2H, int log2W,
                              int mx, int my, float scale, const float2* tw, hipStream_t s) {
    const ModeAddr ma = make_addr(lay);
    switch (log2H * 16 + log2W) {
#define CASE(LH, LW)                                                                                            \
    case LH * 16 + LW: {                                                                                        \
        const size_t lds = SmallPlan<LH, LW>::lds_bytes(my);                                                    \
        hipLaunchKernelGGL((k_inv2d_small<LH, LW>), dim3((unsigned)nimg), dim3(kSmallThreads), lds, s, yh, out, \
                           ma, mx, my, scale, tw);                                                              \
        break;                                                                                                  \
    }
        FNO_SMALL_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fno
