// Fused per-image forward and inverse transforms for grids with H, W <= 128.
//
// Forward (per image): the real rows are transformed two at a time as one
// complex row z = x[p] + i x[p + H/2]; only the bins a truncated row spectrum
// needs (ky < my and their mirrors W - ky) are kept in LDS.  The column pass
// rebuilds each row's half spectrum on the fly (A = (Z[k] + conj Z[-k]) / 2,
// B = (Z[k] - conj Z[-k]) / 2i), transforms the my columns along H and writes
// only kx in [0,mx) u [H-mx,H), scaled.
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
// the R2-point DFTs across t, giving X[k1 + R1 k2].  Rows add one radix-2
// level on top (even and odd samples per thread, see SmallPlan).
//
// Scheduling: a persistent grid of a few workgroups per CU walks the images;
// as soon as a workgroup has moved the current image's global inputs from
// registers into LDS it issues the loads of its next image, which land while
// it finishes the current one (its barriers order LDS only, so those loads
// are not waited for early).  Images are handed
// out so that the workgroups the hardware places on one XCD at the same time
// work on neighbouring channels, whose spectra share 128-byte lines in the
// tiled layout below.
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
constexpr int kSmallBlocksPerCU = 2;

template <int N> struct Split;
template <> struct Split<4>   { static constexpr int R1 = 2,  R2 = 2; };
template <> struct Split<8>   { static constexpr int R1 = 4,  R2 = 2; };
template <> struct Split<16>  { static constexpr int R1 = 4,  R2 = 4; };
template <> struct Split<32>  { static constexpr int R1 = 8,  R2 = 4; };
template <> struct Split<64>  { static constexpr int R1 = 8,  R2 = 8; };
template <> struct Split<128> { static constexpr int R1 = 16, R2 = 8; };

__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }

struct ModeAddr {
    int64_t sb, sc, st;
    int C;
    // address of mode m of image img = b * C + c, relative to the image base
    // (image counts stay below 2^31 on this path: every image has >= 64 points)
    __device__ __forceinline__ int64_t base(int64_t img) const {
        const uint32_t i32 = (uint32_t)img;
        const uint32_t b = i32 / (uint32_t)C;
        const uint32_t c = i32 - b * (uint32_t)C;
        return (int64_t)b * sb + (int64_t)c * sc;
    }
    __device__ __forceinline__ int64_t off(int m) const { return (int64_t)(m >> 3) * st + (m & 7); }
};

// Rows: a complex row of length W is split as n = q + 2 (t + T m) with
// q in {0,1} held in one thread (so every lane moves float2 pairs), t < T
// across the T lanes of the row and m < M in registers (W / 2 = T * M).  The
// even / odd halves (q) get a W/2-point transform each (in-register DFT over
// m, twiddle, LDS hand-over, DFT over t), and one radix-2 step with
// W_W^k joins them.  Columns: n = t + R2 m with R1 = M points per thread.
template <int LOG2H, int LOG2W>
struct SmallPlan {
    static constexpr int H = 1 << LOG2H;
    static constexpr int W = 1 << LOG2W;
    static constexpr int P = H / 2;                 // complex rows (real row pairs)
    static constexpr int MW = Split<W / 2>::R1;     // points per thread and half (q)
    static constexpr int TW = Split<W / 2>::R2;     // lanes per row
    static constexpr int R1H = Split<H>::R1, R2H = Split<H>::R2;
    // LDS exchange: each row (column) group owns T slots of an odd number of
    // complex values.  In the row phase the lanes of a wave are (group, slot)
    // with the slot fastest, so the group stride is made congruent to T
    // modulo 16 double-words; in the column phase the group (column) index is
    // fastest, so that stride is made odd.  Either way the 8-byte accesses of
    // a wave spread over all banks.
    static constexpr int XSW = 2 * MW + 1;
    static constexpr int XSH = R1H + 1;
    static constexpr int GSR = TW * XSW + ((TW - (TW * XSW) % 16) + 16) % 16;
    static constexpr int GSC = R2H * XSH + ((R2H * XSH) % 2 == 0 ? 1 : 0);
    static constexpr int ROWS_IT = kSmallThreads / TW;
    static constexpr int COLS_IT = kSmallThreads / R2H;
    static constexpr int ITERS_R = (P + ROWS_IT - 1) / ROWS_IT;
    static constexpr int XBUF = (ROWS_IT * GSR > COLS_IT * GSC) ? ROWS_IT * GSR : COLS_IT * GSC;
    static_assert(MW >= TW && MW % TW == 0, "row split");
    static_assert(R1H >= R2H && R1H % R2H == 0 && R1H >= 2, "column split");
    // Row stride of the spectrum planes: >= my and congruent to T modulo 16,
    // so the rows written by one wave land on different banks.
    static __host__ __device__ int plane_stride(int my) { return my + ((TW - my % 16) + 16) % 16; }
    // LDS: twiddles for W and H, two spectrum planes of H/2 rows (forward) or
    // one plane of H rows (inverse), and the exchange buffer.
    static size_t lds_bytes(int my) {
        return sizeof(float2) * ((size_t)W + H + (size_t)H * plane_stride(my) + XBUF);
    }
};

// Row batch `it` of image xi: rows a = p and b = p + P, float2 pairs at
// 2 (t + T m).  Rows past P (small grids) load row 0 and are not used.
template <int LOG2H, int LOG2W>
__device__ __forceinline__ void small_load_rows(const float* xi,
                                                float2 (&ba)[SmallPlan<LOG2H, LOG2W>::ITERS_R][SmallPlan<LOG2H, LOG2W>::MW],
                                                float2 (&bb)[SmallPlan<LOG2H, LOG2W>::ITERS_R][SmallPlan<LOG2H, LOG2W>::MW],
                                                int pl, int t) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int W = S::W, P = S::P, MW = S::MW, TW = S::TW, IT = S::ITERS_R;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int p = it * S::ROWS_IT + pl;
        const int pp = p < P ? p : 0;
        const float2* ra = reinterpret_cast<const float2*>(xi + pp * W) + t;
        const float2* rb = reinterpret_cast<const float2*>(xi + (pp + P) * W) + t;
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            ba[it][m] = ra[TW * m];
            bb[it][m] = rb[TW * m];
        }
    }
}

// Row pass of one image (forward): the complex rows p = x[p] + i x[p + P],
// taken from registers (ba, bb), are transformed and the bins a truncated
// row spectrum needs land in the planes zlo (Z_p[k], k < my) and zhi
// (Z_p[(W - k) mod W]).  Ends with a workgroup barrier.
template <int LOG2H, int LOG2W>
__device__ __forceinline__ void small_fwd_rows(const float2 (&ba)[SmallPlan<LOG2H, LOG2W>::ITERS_R][SmallPlan<LOG2H, LOG2W>::MW],
                                               const float2 (&bb)[SmallPlan<LOG2H, LOG2W>::ITERS_R][SmallPlan<LOG2H, LOG2W>::MW],
                                               float2* zlo, float2* zhi, int ms, int my, const float2* twW, float2* xbr,
                                               int pl, int t) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int W = S::W, P = S::P, MW = S::MW, TW = S::TW, IT = S::ITERS_R;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int p = it * S::ROWS_IT + pl;
        const bool active = p < P;
        if (active) {
            float2 c0[MW], c1[MW];         // even (q = 0) and odd (q = 1) samples
#pragma unroll
            for (int m = 0; m < MW; ++m) {
                c0[m] = make_float2(ba[it][m].x, bb[it][m].x);
                c1[m] = make_float2(ba[it][m].y, bb[it][m].y);
            }
            dft<MW, -1>(c0);
            dft<MW, -1>(c1);
#pragma unroll
            for (int k1 = 1; k1 < MW; ++k1) {
                const float2 w = twW[(2 * t * k1) & (W - 1)];   // W_{W/2}^{t k1}
                c0[k1] = cmul(c0[k1], w);
                c1[k1] = cmul(c1[k1], w);
            }
#pragma unroll
            for (int k1 = 0; k1 < MW; ++k1) {
                xbr[t * S::XSW + k1] = c0[k1];
                xbr[t * S::XSW + MW + k1] = c1[k1];
            }
        }
        lds_barrier();
        if (active) {
#pragma unroll
            for (int jj = 0; jj < MW / TW; ++jj) {
                const int k1 = t + TW * jj;
                float2 u0[TW], u1[TW];
#pragma unroll
                for (int tt = 0; tt < TW; ++tt) {
                    u0[tt] = xbr[tt * S::XSW + k1];
                    u1[tt] = xbr[tt * S::XSW + MW + k1];
                }
                dft<TW, -1>(u0);
                dft<TW, -1>(u1);
#pragma unroll
                for (int k2 = 0; k2 < TW; ++k2) {
                    const int kh = k1 + MW * k2;                    // < W/2
                    const float2 y1 = cmul(u1[k2], twW[kh]);
                    const float2 lo = cadd(u0[k2], y1);             // Z[kh]
                    const float2 hi = csub(u0[k2], y1);             // Z[kh + W/2]
                    if (kh < my) zlo[p * ms + kh] = lo;
                    const int kml = (W - kh) & (W - 1);
                    if (kml < my) zhi[p * ms + kml] = lo;
                    const int khh = kh + W / 2;
                    if (khh < my) zlo[p * ms + khh] = hi;
                    const int kmh = W / 2 - kh;                     // (W - khh) mod W
                    if (kmh < my) zhi[p * ms + kmh] = hi;
                }
            }
        }
        lds_barrier();
    }
}

// Column pass of one image (forward): each row's half spectrum is rebuilt
// from the planes, the my columns are transformed along H and every kept
// mode m = q my + ky goes out through store(m, value) (unscaled).  Ends with
// a workgroup barrier.
template <int LOG2H, int LOG2W, typename Store>
__device__ __forceinline__ void small_fwd_cols(const float2* zlo, const float2* zhi, int ms, int mx, int my,
                                               const float2* twH, float2* xbc, int tc, int cl, Store&& store) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int H = S::H, R1H = S::R1H, R2H = S::R2H;
    const int ky = cl;
    const bool active = ky < my;
    if (active) {
        float2 v[R1H];
#pragma unroll
        for (int m = 0; m < R1H / 2; ++m) {
            const int p = tc + R2H * m;
            const float2 zl = zlo[p * ms + ky];
            const float2 zm = zhi[p * ms + ky];
            v[m] = make_float2(0.5f * (zl.x + zm.x), 0.5f * (zl.y - zm.y));
            v[m + R1H / 2] = make_float2(0.5f * (zl.y + zm.y), -0.5f * (zl.x - zm.x));
        }
        dft<R1H, -1>(v);
#pragma unroll
        for (int k1 = 1; k1 < R1H; ++k1) v[k1] = cmul(v[k1], twH[(tc * k1) & (H - 1)]);
#pragma unroll
        for (int k1 = 0; k1 < R1H; ++k1) xbc[tc * S::XSH + k1] = v[k1];
    }
    lds_barrier();
    if (active) {
#pragma unroll
        for (int j = 0; j < R1H / R2H; ++j) {
            const int k1 = tc + R2H * j;
            float2 u[R2H];
#pragma unroll
            for (int tt = 0; tt < R2H; ++tt) u[tt] = xbc[tt * S::XSH + k1];
            dft<R2H, -1>(u);
#pragma unroll
            for (int k2 = 0; k2 < R2H; ++k2) {
                const int kx = k1 + R1H * k2;
                const int q = kx < mx ? kx : (kx >= H - mx ? kx - H + 2 * mx : -1);
                if (q >= 0) store(q * my + ky, u[k2]);
            }
        }
    }
    lds_barrier();
}

template <int LOG2H, int LOG2W>
__global__ __launch_bounds__(kSmallThreads, kSmallBlocksPerCU) void k_fwd2d_small(
    const float* __restrict__ x, float2* __restrict__ xh, ModeAddr ma, int64_t nimg, int mx_arg, int my_arg,
    float scale, const float2* __restrict__ tw) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int H = S::H, W = S::W, P = S::P;
    constexpr int MW = S::MW, TW = S::TW;
    constexpr int IT = S::ITERS_R;
    extern __shared__ float2 smem[];
    float2* twW = smem;
    float2* twH = twW + W;
    // zlo = [P][ms]: Z_p[k], k < my; zhi = [P][ms]: Z_p[(W - k) mod W]
    float2* zplanes = twH + H;
    float2* xbuf = zplanes + 2 * P * S::plane_stride(my_arg);

    const int tid = threadIdx.x;
    for (int j = tid; j < W; j += kSmallThreads) twW[j] = tw[j * (kNMax / W)];
    for (int j = tid; j < H; j += kSmallThreads) twH[j] = tw[j * (kNMax / H)];
    lds_barrier();

    const int pl = tid / TW;             // row-pass role
    const int t = tid % TW;
    const int tc = tid / S::COLS_IT;     // column-pass role
    const int cl = tid % S::COLS_IT;
    float2* xbr = xbuf + pl * S::GSR;
    float2* xbc = xbuf + cl * S::GSC;

    auto load = [&](int64_t img, float2 (&ba)[IT][MW], float2 (&bb)[IT][MW]) {
        small_load_rows<LOG2H, LOG2W>(x + img * (int64_t)(H * W), ba, bb, pl, t);
    };

    const int64_t G = gridDim.x;
    int64_t L = blockIdx.x;
    float2 ba[IT][MW], bb[IT][MW];
    load(paired_image(L, nimg), ba, bb);
    while (true) {
        const int64_t img = paired_image(L, nimg);
        const int64_t Ln = L + G;
        // Opaque per-image copies of the mode counts: everything derived from
        // them (predicates, LDS and output offsets) is recomputed per image
        // instead of being hoisted out of the loop into ~100 live registers.
        int my = my_arg, mx = mx_arg;
        asm volatile("" : "+s"(my), "+s"(mx));
        const int ms = S::plane_stride(my);
        float2* zlo = zplanes;
        float2* zhi = zplanes + P * ms;
        // ---- rows: complex row p = x[p] + i x[p + P] ----------------------
        small_fwd_rows<LOG2H, LOG2W>(ba, bb, zlo, zhi, ms, my, twW, xbr, pl, t);

        // the register buffer is free once every row batch has gone through
        // LDS: start fetching the next image, it lands during the column pass
        // (the empty asm keeps the compiler from hoisting these loads into
        // the row pass, where the current image's registers are still live)
        asm volatile("" ::: "memory");
        if (Ln < nimg) load(paired_image(Ln, nimg), ba, bb);

        // ---- columns ky < my along H, kept kx only (one batch: my <= COLS_IT)
        const int64_t obase = ma.base(img);
        small_fwd_cols<LOG2H, LOG2W>(zlo, zhi, ms, mx, my, twH, xbc, tc, cl, [&](int m, float2 v) {
            xh[obase + ma.off(m)] = cscale(v, scale);
        });
        L = Ln;
        if (L >= nimg) break;
    }
}

// Column pass of one image (inverse): R'[h][ky] = sum over the kept kx of
// Y[kx][ky] W_H^{+h kx}, from the gathered inputs pre (dropped kx zeroed
// here) into the plane rp.  mid() runs once the gathered registers are free
// (the persistent kernel fetches its next image there).  Ends with a
// workgroup barrier.
template <int LOG2H, int LOG2W, typename Mid>
__device__ __forceinline__ void small_inv_cols(
    const float2 (&pre)[SmallPlan<LOG2H, LOG2W>::R1H / SmallPlan<LOG2H, LOG2W>::R2H][SmallPlan<LOG2H, LOG2W>::R2H],
    float2* rp, int ms, int mx, int my, const float2* twH, float2* xbc, int tc, int cl, Mid&& mid) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int H = S::H, R1H = S::R1H, R2H = S::R2H, KJ = R1H / R2H;
    const int ky = cl;
    const bool active = ky < my;
    if (active) {
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int k1 = tc + R2H * j;
            float2 u[R2H];
#pragma unroll
            for (int k2 = 0; k2 < R2H; ++k2) {
                const int kx = k1 + R1H * k2;
                const bool kept = kx < mx || kx >= H - mx;
                u[k2] = kept ? pre[j][k2] : make_float2(0.0f, 0.0f);
            }
            dft<R2H, +1>(u);
#pragma unroll
            for (int tt = 1; tt < R2H; ++tt) u[tt] = cmul(u[tt], conjf2(twH[(tt * k1) & (H - 1)]));
#pragma unroll
            for (int tt = 0; tt < R2H; ++tt) xbc[tt * S::XSH + k1] = u[tt];
        }
    }
    mid();
    lds_barrier();
    if (active) {
        float2 v[R1H];
#pragma unroll
        for (int k1 = 0; k1 < R1H; ++k1) v[k1] = xbc[tc * S::XSH + k1];
        dft<R1H, +1>(v);
#pragma unroll
        for (int m = 0; m < R1H; ++m) rp[(tc + R2H * m) * ms + ky] = v[m];
    }
    lds_barrier();
}

// Row pass of one image (inverse): two real rows per complex inverse
// transform, Z = Ya_herm + i Yb_herm (imaginary parts of DC / Nyquist
// dropped); even / odd outputs q: S_q[k] = (Z[k] +- Z[k + W/2]) W_W^{+q k}.
// out(p, m, a, b) receives, unscaled, the float2 pair at 2 (t + T m) of row
// p (a) and of row p + P (b).  Ends with a workgroup barrier.
template <int LOG2H, int LOG2W, typename Out>
__device__ __forceinline__ void small_inv_rows(const float2* rp, int ms, int my, const float2* twW, float2* xbr, int pl,
                                               int t, Out&& out) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int W = S::W, P = S::P, MW = S::MW, TW = S::TW;
#pragma unroll
    for (int it = 0; it < S::ITERS_R; ++it) {
        const int p = it * S::ROWS_IT + pl;
        const bool active = p < P;
        if (active) {
            const float2* ya_row = rp + p * ms;
            const float2* yb_row = rp + (p + P) * ms;
            auto zin = [&](int k) {
                const int kk = k <= W / 2 ? k : W - k;
                float2 z = make_float2(0.0f, 0.0f);
                if (kk < my) {
                    const float2 ya = ya_row[kk];
                    const float2 yb = yb_row[kk];
                    if (kk == 0 || 2 * kk == W) z = make_float2(ya.x, yb.x);
                    else if (k == kk) z = make_float2(ya.x - yb.y, ya.y + yb.x);
                    else z = make_float2(ya.x + yb.y, yb.x - ya.y);
                }
                return z;
            };
#pragma unroll
            for (int jj = 0; jj < MW / TW; ++jj) {
                const int k1 = t + TW * jj;
                float2 u0[TW], u1[TW];
#pragma unroll
                for (int k2 = 0; k2 < TW; ++k2) {
                    const int kh = k1 + MW * k2;                    // < W/2
                    const float2 zl = zin(kh);
                    const float2 zh = zin(kh + W / 2);
                    u0[k2] = cadd(zl, zh);
                    u1[k2] = cmul(csub(zl, zh), conjf2(twW[kh]));
                }
                dft<TW, +1>(u0);
                dft<TW, +1>(u1);
#pragma unroll
                for (int tt = 0; tt < TW; ++tt) {
                    const float2 w = conjf2(twW[(2 * tt * k1) & (W - 1)]);   // W_{W/2}^{+tt k1}
                    xbr[tt * S::XSW + k1] = cmul(u0[tt], w);
                    xbr[tt * S::XSW + MW + k1] = cmul(u1[tt], w);
                }
            }
        }
        lds_barrier();
        if (active) {
            float2 v0[MW], v1[MW];
#pragma unroll
            for (int k1 = 0; k1 < MW; ++k1) {
                v0[k1] = xbr[t * S::XSW + k1];
                v1[k1] = xbr[t * S::XSW + MW + k1];
            }
            dft<MW, +1>(v0);
            dft<MW, +1>(v1);
#pragma unroll
            for (int m = 0; m < MW; ++m) out(p, m, make_float2(v0[m].x, v1[m].x), make_float2(v0[m].y, v1[m].y));
        }
        lds_barrier();
    }
}

// EPI: the fused output epilogue (bias, GELU, second branch) on every
// output pair, the branch read at the same index.
template <int LOG2H, int LOG2W, bool EPI>
__global__ __launch_bounds__(kSmallThreads, kSmallBlocksPerCU) void k_inv2d_small(
    const float2* __restrict__ yh, float* __restrict__ out, ModeAddr ma, int64_t nimg, int mx_arg, int my_arg,
    float scale, const float2* __restrict__ tw, Epilogue epi) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int H = S::H, W = S::W, P = S::P;
    constexpr int TW = S::TW, R1H = S::R1H, R2H = S::R2H;
    constexpr int KJ = R1H / R2H;
    extern __shared__ float2 smem[];
    float2* twW = smem;
    float2* twH = twW + W;
    float2* rp = twH + H;               // [H][ms]: column-inverted spectrum R'[h][ky]
    float2* xbuf = rp + H * S::plane_stride(my_arg);

    const int tid = threadIdx.x;
    for (int j = tid; j < W; j += kSmallThreads) twW[j] = tw[j * (kNMax / W)];
    for (int j = tid; j < H; j += kSmallThreads) twH[j] = tw[j * (kNMax / H)];
    lds_barrier();

    const int pl = tid / TW;
    const int t = tid % TW;
    const int tc = tid / S::COLS_IT;
    const int cl = tid % S::COLS_IT;
    const int kyc = cl < my_arg ? cl : 0;    // column this thread gathers (dummy 0 when idle)
    float2* xbr = xbuf + pl * S::GSR;
    float2* xbc = xbuf + cl * S::GSC;

    // Inputs of this thread's column batch: Y[kx][ky] at kx = k1 + R1H k2.
    // Loads are unconditional (dropped kx read mode 0) so the prefetch never
    // forces an early wait; dropped values are zeroed where they are used.
    auto gather = [&](int64_t img, float2 (&u)[KJ][R2H]) {
        int my = my_arg, mx = mx_arg;
        asm volatile("" : "+s"(my), "+s"(mx));
        const int64_t ibase = ma.base(img);
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int k1 = tc + R2H * j;
#pragma unroll
            for (int k2 = 0; k2 < R2H; ++k2) {
                const int kx = k1 + R1H * k2;
                const int q = kx < mx ? kx : (kx >= H - mx ? kx - H + 2 * mx : -1);
                const int mode = q >= 0 ? q * my + kyc : 0;
                u[j][k2] = yh[ibase + ma.off(mode)];
            }
        }
    };

    const int64_t G = gridDim.x;
    int64_t L = blockIdx.x;
    float2 pre[KJ][R2H];
    gather(paired_image(L, nimg), pre);
    while (true) {
        const int64_t img = paired_image(L, nimg);
        const int64_t Ln = L + G;
        // opaque per-image copies of the mode counts (see the forward kernel)
        int my = my_arg, mx = mx_arg;
        asm volatile("" : "+s"(my), "+s"(mx));
        const int ms = S::plane_stride(my);
        // ---- columns: R'[h][ky] = sum_{kept kx} Y[kx][ky] W_H^{+h kx} -------
        // (one batch: my <= COLS_IT on this path); the prefetch registers are
        // free once the column inputs are in LDS: fetch the next image's
        small_inv_cols<LOG2H, LOG2W>(pre, rp, ms, mx, my, twH, xbc, tc, cl, [&]() {
            asm volatile("" ::: "memory");
            if (Ln < nimg) gather(paired_image(Ln, nimg), pre);
        });

        // ---- rows: two real rows per complex inverse transform -------------
        float* oi = out + img * (int64_t)(H * W);
        if constexpr (EPI) {
            // the image's branch through a buffer resource (an empty range for
            // a null branch reads zero)
            const float bias = epi_bias(epi, (uint32_t)img);
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(epi.branch ? epi.branch + img * (int64_t)(H * W) : nullptr,
                                                        epi.branch ? (uint32_t)(H * W * 4) : 0u);
            small_inv_rows<LOG2H, LOG2W>(rp, ms, my, twW, xbr, pl, t, [&](int p, int m, float2 a, float2 b) {
                const uint32_t col = (uint32_t)(2 * (t + TW * m));
                const float2 za = buffer_load_f2(rb, (uint32_t)((p * W) + col) * 4u, 0);
                const float2 zb = buffer_load_f2(rb, (uint32_t)(((p + P) * W) + col) * 4u, 0);
                float2* oa = reinterpret_cast<float2*>(oi + p * W) + t;
                float2* ob = reinterpret_cast<float2*>(oi + (p + P) * W) + t;
                nt_store2(&oa[TW * m], make_float2(epi_apply(epi, a.x * scale, bias, za.x),
                                                   epi_apply(epi, a.y * scale, bias, za.y)));
                nt_store2(&ob[TW * m], make_float2(epi_apply(epi, b.x * scale, bias, zb.x),
                                                   epi_apply(epi, b.y * scale, bias, zb.y)));
            });
        } else {
            small_inv_rows<LOG2H, LOG2W>(rp, ms, my, twW, xbr, pl, t, [&](int p, int m, float2 a, float2 b) {
                float2* oa = reinterpret_cast<float2*>(oi + p * W) + t;
                float2* ob = reinterpret_cast<float2*>(oi + (p + P) * W) + t;
                nt_store2(&oa[TW * m], make_float2(a.x * scale, a.y * scale));
                nt_store2(&ob[TW * m], make_float2(b.x * scale, b.y * scale));
            });
        }
        L = Ln;
        if (L >= nimg) break;
    }
}

// The whole call for small problems in one kernel, one workgroup per batch
// item (TurboFNO blog, sections 2.1-2.2 and 3.2 "Section 3": forward
// transform, channel mix and inverse in one kernel, the truncated spectrum
// kept on chip).  NG groups of 256 threads transform NG channel images at a
// time with the per-image code above; the batch item's truncated spectra
// X[b] (Cin x M) and Y[b] (Cout x M, M = 2 mx my) stay in LDS, and the mix
// Y[o][m] = sum_i X[i][m] W[m][i][o] runs between two workgroup barriers.
// Every group runs the same number of rounds (idle groups redo the last
// channel and store nothing), so the workgroup barriers inside the
// per-image code stay matched.
template <int LOG2H, int LOG2W, int NG>
__global__ __launch_bounds__(kSmallThreads * NG) void k_conv2d_small_fused(
    const float* __restrict__ x, const float2* __restrict__ w, float* __restrict__ out, int Cin, int Cout, int mx,
    int my, float scale, const float2* __restrict__ tw) {
    using S = SmallPlan<LOG2H, LOG2W>;
    constexpr int H = S::H, W = S::W, P = S::P, MW = S::MW, TW = S::TW, IT = S::ITERS_R;
    constexpr int R1H = S::R1H, R2H = S::R2H, KJ = R1H / R2H;
    extern __shared__ float2 smem[];
    const int M = 2 * mx * my;
    const int ms = S::plane_stride(my);
    float2* twW = smem;
    float2* twH = twW + W;
    float2* xs = twH + H;                       // [Cin][M]
    float2* ys = xs + Cin * M;                  // [Cout][M]
    const int g = threadIdx.x / kSmallThreads;  // image group
    const int tid = threadIdx.x % kSmallThreads;
    // the group's planes and exchange buffer: forward Z planes, later the
    // inverse's R' plane
    float2* reg = ys + Cout * M + g * (H * ms + S::XBUF);
    float2* xbuf = reg + H * ms;
    for (int j = threadIdx.x; j < W; j += kSmallThreads * NG) twW[j] = tw[j * (kNMax / W)];
    for (int j = threadIdx.x; j < H; j += kSmallThreads * NG) twH[j] = tw[j * (kNMax / H)];
    lds_barrier();

    const int pl = tid / TW;             // row-pass role
    const int t = tid % TW;
    const int tc = tid / S::COLS_IT;     // column-pass role
    const int cl = tid % S::COLS_IT;
    float2* xbr = xbuf + pl * S::GSR;
    float2* xbc = xbuf + cl * S::GSC;
    const int64_t b = blockIdx.x;

    // ---- forward transforms of the batch item's Cin images -----------------
    for (int c0 = 0; c0 < Cin; c0 += NG) {
        const int c = c0 + g;
        const bool on = c < Cin;
        const int cc = on ? c : Cin - 1;
        float2 ba[IT][MW], bb[IT][MW];
        small_load_rows<LOG2H, LOG2W>(x + (b * Cin + cc) * (int64_t)(H * W), ba, bb, pl, t);
        small_fwd_rows<LOG2H, LOG2W>(ba, bb, reg, reg + P * ms, ms, my, twW, xbr, pl, t);
        small_fwd_cols<LOG2H, LOG2W>(reg, reg + P * ms, ms, mx, my, twH, xbc, tc, cl, [&](int m, float2 v) {
            if (on) xs[cc * M + m] = cscale(v, scale);
        });
    }

    // ---- channel mix in LDS -------------------------------------------------
    for (int e = threadIdx.x; e < Cout * M; e += kSmallThreads * NG) {
        const int o = e % Cout, m = e / Cout;
        const float2* wm = w + (int64_t)m * Cin * Cout + o;
        float2 acc = make_float2(0.0f, 0.0f);
        for (int i = 0; i < Cin; ++i) acc = cfma(acc, xs[i * M + m], wm[(int64_t)i * Cout]);
        ys[o * M + m] = acc;
    }
    lds_barrier();

    // ---- inverse transforms of the Cout output images -----------------------
    const int kyc = cl < my ? cl : 0;
    for (int o0 = 0; o0 < Cout; o0 += NG) {
        const int o = o0 + g;
        const bool on = o < Cout;
        const int oc = on ? o : Cout - 1;
        float2 pre[KJ][R2H];
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int k1 = tc + R2H * j;
#pragma unroll
            for (int k2 = 0; k2 < R2H; ++k2) {
                const int kx = k1 + R1H * k2;
                const int q = kx < mx ? kx : (kx >= H - mx ? kx - H + 2 * mx : -1);
                pre[j][k2] = ys[oc * M + (q >= 0 ? q * my + kyc : 0)];
            }
        }
        small_inv_cols<LOG2H, LOG2W>(pre, reg, ms, mx, my, twH, xbc, tc, cl, []() {});
        float* oi = out + (b * Cout + oc) * (int64_t)(H * W);
        small_inv_rows<LOG2H, LOG2W>(reg, ms, my, twW, xbr, pl, t, [&](int p, int m, float2 a, float2 bv) {
            if (!on) return;
            float2* oa = reinterpret_cast<float2*>(oi + p * W) + t;
            float2* ob = reinterpret_cast<float2*>(oi + (p + P) * W) + t;
            oa[TW * m] = make_float2(a.x * scale, a.y * scale);
            ob[TW * m] = make_float2(bv.x * scale, bv.y * scale);
        });
    }
}

constexpr int kFusedMaxChannels = 8;   // channels in and out: at most two rounds of four images
constexpr int kFusedGroups = 4;        // image groups of 256 threads per workgroup
// Grids of at most 1024 points: the four groups' planes and the spectra fit
// the LDS (at 64 x 64 with two groups the one-kernel call measured twice the
// three-kernel time, so larger grids keep the three kernels).
constexpr int kFusedMaxLog2Points = 10;

template <int LH, int LW>
size_t fused_lds_bytes(int Cin, int Cout, int mx, int my) {
    using S = SmallPlan<LH, LW>;
    constexpr int NG = kFusedGroups;
    return sizeof(float2) * ((size_t)S::W + S::H + (size_t)(Cin + Cout) * 2 * mx * my +
                             (size_t)NG * ((size_t)S::H * S::plane_stride(my) + S::XBUF));
}

#define FNO_FUSED_CASES(MACRO) \
    MACRO(3, 3) MACRO(3, 4) MACRO(3, 5) MACRO(3, 6) MACRO(3, 7) \
    MACRO(4, 3) MACRO(4, 4) MACRO(4, 5) MACRO(4, 6) \
    MACRO(5, 3) MACRO(5, 4) MACRO(5, 5) \
    MACRO(6, 3) MACRO(6, 4) \
    MACRO(7, 3)

size_t fused_lds_for(int log2H, int log2W, int Cin, int Cout, int mx, int my) {
    switch (log2H * 16 + log2W) {
#define CASE(LH, LW) \
    case LH * 16 + LW: return fused_lds_bytes<LH, LW>(Cin, Cout, mx, my);
        FNO_FUSED_CASES(CASE)
#undef CASE
        default: return (size_t)-1;
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

// Persistent grid: a multiple of 16 workgroups (see paired_image), at most
// kSmallBlocksPerCU per CU, never more than there are images.
unsigned persistent_grid(int64_t nimg) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    int64_t g = (int64_t)cus * kSmallBlocksPerCU;
    g = (g / 16) * 16;
    if (g < 16) g = 16;
    if (g > nimg) g = nimg;
    return (unsigned)g;
}

}  // namespace

bool small2d_supported(int log2H, int log2W, int my) {
    if (log2H < 3 || log2H > 7 || log2W < 3 || log2W > 7) return false;
    // the my kept columns must fit one column batch of the workgroup
    const int r2h = log2H == 3 ? 2 : log2H <= 5 ? 4 : 8;
    if (my > kSmallThreads / r2h) return false;
    const size_t need = sizeof(float2) * ((size_t)(1 << log2W) + (1 << log2H) + (size_t)(1 << log2H) * (my + 16) +
                                          256 * 18);
    return need <= 150 * 1024;
}

hipError_t launch_fwd2d_small(const float* x, float2* xh, const SpecLayout& lay, int64_t nimg, int log2H, int log2W,
                              int mx, int my, float scale, const float2* tw, hipStream_t s) {
    const ModeAddr ma = make_addr(lay);
    const dim3 grid(persistent_grid(nimg));
    switch (log2H * 16 + log2W) {
#define CASE(LH, LW)                                                                                          \
    case LH * 16 + LW: {                                                                                      \
        const size_t lds = SmallPlan<LH, LW>::lds_bytes(my);                                                  \
        return launch_kernel((k_fwd2d_small<LH, LW>), grid, dim3(kSmallThreads), lds, s, x, xh, ma, nimg, mx, my, \
                           scale, tw);                                                                        \
    }
        FNO_SMALL_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
}

bool conv2d_small_fused_supported(int64_t B, int64_t Cin, int64_t Cout, int log2H, int log2W, int mx, int my) {
    if (log2H < 3 || log2W < 3 || log2H + log2W > kFusedMaxLog2Points || !small2d_supported(log2H, log2W, my))
        return false;
    if (B < 1 || B > 65535 || Cin < 1 || Cin > kFusedMaxChannels || Cout < 1 || Cout > kFusedMaxChannels) return false;
    return fused_lds_for(log2H, log2W, (int)Cin, (int)Cout, mx, my) <= 160 * 1024;
}

hipError_t launch_conv2d_small_fused(const float* x, const float2* w, float* out, int64_t B, int64_t Cin, int64_t Cout,
                                     int log2H, int log2W, int mx, int my, float scale, const float2* tw,
                                     hipStream_t s) {
    if (!conv2d_small_fused_supported(B, Cin, Cout, log2H, log2W, mx, my)) return hipErrorInvalidValue;
    const size_t lds = fused_lds_for(log2H, log2W, (int)Cin, (int)Cout, mx, my);
    const dim3 grid((unsigned)B);
    const int iCin = (int)Cin, iCout = (int)Cout;
    switch (log2H * 16 + log2W) {
#define CASE(LH, LW)                                                                                            \
    case LH * 16 + LW: {                                                                                        \
        constexpr int NG = kFusedGroups;                                                                        \
        return launch_kernel((k_conv2d_small_fused<LH, LW, NG>), grid, dim3(kSmallThreads * NG), lds, s, x, w, out, \
                             iCin, iCout, mx, my, scale, tw);                                                   \
    }
        FNO_FUSED_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_inv2d_small(const float2* yh, float* out, const SpecLayout& lay, int64_t nimg, int log2H, int log2W,
                              int mx, int my, float scale, const float2* tw, hipStream_t s, const Epilogue& epi) {
    const ModeAddr ma = make_addr(lay);
    const dim3 grid(persistent_grid(nimg));
    switch (log2H * 16 + log2W) {
#define CASE(LH, LW)                                                                                              \
    case LH * 16 + LW: {                                                                                          \
        const size_t lds = SmallPlan<LH, LW>::lds_bytes(my);                                                      \
        if (epi.on)                                                                                               \
            return launch_kernel((k_inv2d_small<LH, LW, true>), grid, dim3(kSmallThreads), lds, s, yh, out, ma,   \
                                 nimg, mx, my, scale, tw, epi);                                                   \
        return launch_kernel((k_inv2d_small<LH, LW, false>), grid, dim3(kSmallThreads), lds, s, yh, out, ma, nimg, \
                             mx, my, scale, tw, epi);                                                             \
    }
        FNO_SMALL_CASES(CASE)
#undef CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fno
