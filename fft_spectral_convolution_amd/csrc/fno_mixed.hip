// Stage kernels for transform lengths that are not powers of two: any
// 7-smooth N (2^a 3^b 5^c 7^d) from 2 to 4096, and for the rows alone up to
// 8192 (the padded rows of a linear convolution) (the FFT blog, section 6.2:
// sizes such as 96 or 100 take mixed-radix paths; section 2.1: the padded
// length of a linear convolution).  Same contracts as the generic
// power-of-two stage kernels (fno_generic.hip), with the transform run as
// a mixed-radix Stockham FFT in LDS (radix-4/2 passes first, then 3, 5, 7)
// on a per-length twiddle table W_N^m = exp(-2 pi i m / N), m < N, built on
// the host in double precision and rounded once.
#include <cmath>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kMrThreads = 1024;   // 16 waves; the 72 KiB of LDS allow two workgroups per CU
constexpr int kMrMaxPasses = 12;
constexpr int kMrTwLds = 1024;     // lengths up to this take their twiddle table from LDS
// Rows longer than kLdsElems (up to kMrLongRow points: the padded rows of a
// linear convolution) take workgroups with one 8192-point buffer and
// in-place passes (64 KiB of LDS, one pair of rows per workgroup, two
// workgroups per CU).
constexpr int kMrLongRow = 8192;

// Passes of an n-point transform: radix r[p], J = n / r[p] butterflies per
// row, ns[p] = product of the earlier radices, twiddle step n / (ns r); the
// reciprocals of J and ns for qdiv.
struct MRPlan {
    int n, npass;
    int r[kMrMaxPasses], j[kMrMaxPasses], ns[kMrMaxPasses], step[kMrMaxPasses];
    float inv_j[kMrMaxPasses], inv_ns[kMrMaxPasses];
};

// floor(x / d) for 0 <= x < 2^21, from inv = 1/d rounded to float (or within
// one ulp of it): (x + 1/2) / d lies at least 1/(2d) from every integer,
// and the product's relative error (below 2^-22) moves it by less than that.
// All the index arithmetic here is below 2^13.
__device__ __forceinline__ int qdiv(int x, float inv) { return (int)(((float)x + 0.5f) * inv); }

// Radix-R DFT (R = 3, 5, 7), compile-time twiddles:
// v[k] <- sum_r v[r] exp(SIGN 2 pi i r k / R).  The terms r and R - r are
// taken together: with p_r = v[r] + v[R-r], m_r = v[r] - v[R-r] and
// theta = 2 pi r k / R,
//   X[k] = v[0] + sum_{r <= (R-1)/2} (p_r cos theta + i SIGN m_r sin theta),
// and X[R - k] is the same with the sine terms negated: 4 ((R-1)/2)^2 fused
// multiply-adds for the non-zero bins instead of 4 (R-1)^2.
template <int R, int SIGN>
__device__ __forceinline__ void dft_odd(float2 (&v)[R]) {
    constexpr int NH = (R - 1) / 2;
    float2 sp[NH], sm[NH];
    static_for<0, NH>([&](auto t) {
        sp[t] = cadd(v[t + 1], v[R - 1 - t]);
        sm[t] = csub(v[t + 1], v[R - 1 - t]);
    });
    float2 out[R];
    out[0] = v[0];
    static_for<0, NH>([&](auto t) { out[0] = cadd(out[0], sp[t]); });
    static_for<1, NH + 1>([&](auto k) {
        float2 a = v[0], b = make_float2(0.0f, 0.0f);
        static_for<0, NH>([&](auto t) {
            constexpr int e = (k * (t + 1)) % R;
            constexpr float c = (float)exact_cos(8 * e, 8 * R);
            constexpr float s = (float)(SIGN * exact_sin(8 * e, 8 * R));
            a.x = fmaf(sp[t].x, c, a.x);
            a.y = fmaf(sp[t].y, c, a.y);
            b.x = fmaf(sm[t].x, s, b.x);
            b.y = fmaf(sm[t].y, s, b.y);
        });
        out[k] = make_float2(a.x - b.y, a.y + b.x);          // a + i b
        out[R - k] = make_float2(a.x + b.y, a.y - b.x);      // a - i b
    });
#pragma unroll
    for (int k = 0; k < R; ++k) v[k] = out[k];
}

// One radix-R Stockham pass of an n-point transform whose sub-transforms of
// length ns are done: butterfly j reads src[j + r n/R], twiddles by
// W_{ns R}^{r (j mod ns)} (= W_n^{r (j mod ns) step}, step = n / (ns R)),
// runs the radix-R DFT and writes dst[(j - j mod ns) R + j mod ns + r ns].
template <int R, int SIGN>
__device__ __forceinline__ void mr_pass(const float2* src, float2* dst, int stride, int ns, float inv_ns, int step,
                                        int j, const float2* tws) {
    float2 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = src[j + r * stride];
    const int k = j - qdiv(j, inv_ns) * ns;
    if (ns > 1) {
#pragma unroll
        for (int r = 1; r < R; ++r) {
            float2 t = tws[r * k * step];
            if (SIGN > 0) t.y = -t.y;
            v[r] = cmul(v[r], t);
        }
    }
    if constexpr (R == 2 || R == 4) dft<R, SIGN>(v);
    else dft_odd<R, SIGN>(v);
    const int base = (j - k) * R + k;
#pragma unroll
    for (int r = 0; r < R; ++r) dst[base + r * ns] = v[r];
}

// Full transform of `nrows` rows of length p.n (row pitch ld >= p.n) in LDS
// buffer a, ping-ponging through b; returns the buffer with the result.
// tws: the twiddle table, in LDS or global memory.
template <int SIGN>
__device__ __forceinline__ float2* fft_rows_mr(float2* a, float2* b, int nrows, int ld, const MRPlan& p,
                                               const float2* tws, int tid) {
    for (int pass = 0; pass < p.npass; ++pass) {
        const int R = p.r[pass], J = p.j[pass], ns = p.ns[pass], step = p.step[pass];
        const float inv_j = p.inv_j[pass], inv_ns = p.inv_ns[pass];
        const int total = nrows * J;
        // one loop per radix (the radix is uniform over the pass)
        auto run = [&](auto rc) __attribute__((always_inline)) {
            constexpr int RC = decltype(rc)::value;
            for (int idx = tid; idx < total; idx += kMrThreads) {
                const int row = qdiv(idx, inv_j);
                const int j = idx - row * J;
                mr_pass<RC, SIGN>(a + row * ld, b + row * ld, J, ns, inv_ns, step, j, tws);
            }
        };
        switch (R) {
            case 4: run(std::integral_constant<int, 4>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            case 5: run(std::integral_constant<int, 5>{}); break;
            default: run(std::integral_constant<int, 7>{}); break;
        }
        __syncthreads();
        float2* t = a;
        a = b;
        b = t;
    }
    return a;
}

// In-place form for rows longer than kLdsElems (one LDS buffer, so that two
// workgroups fit a CU): in each pass every thread first loads the inputs of
// all its butterflies (at most MB) into registers, the workgroup waits, and
// then every thread writes its outputs (the Stockham output order).  The
// rows hold at most NE elements (nrows * n <= NE), so a radix-R pass has at
// most NE / R butterflies: MB = ceil(NE / (R kMrThreads)) per thread.
template <int SIGN, int NE>
__device__ __forceinline__ void fft_rows_mr_inplace(float2* a, int nrows, int ld, const MRPlan& p, const float2* tws,
                                                    int tid) {
    for (int pass = 0; pass < p.npass; ++pass) {
        const int R = p.r[pass], J = p.j[pass], ns = p.ns[pass], step = p.step[pass];
        const float inv_j = p.inv_j[pass], inv_ns = p.inv_ns[pass];
        const int total = nrows * J;
        auto run = [&](auto rc) __attribute__((always_inline)) {
            constexpr int RC = decltype(rc)::value;
            constexpr int MB = (NE + RC * kMrThreads - 1) / (RC * kMrThreads);
            float2 v[MB][RC];
            int jb[MB], rb[MB];
#pragma unroll
            for (int bi = 0; bi < MB; ++bi) {
                const int idx = tid + bi * kMrThreads;
                jb[bi] = -1;
                rb[bi] = 0;
                if (idx < total) {
                    const int row = qdiv(idx, inv_j);
                    const int j = idx - row * J;
                    rb[bi] = row;
                    jb[bi] = j;
#pragma unroll
                    for (int r = 0; r < RC; ++r) v[bi][r] = a[row * ld + j + r * J];
                }
            }
            __syncthreads();
#pragma unroll
            for (int bi = 0; bi < MB; ++bi) {
                const int j = jb[bi];
                if (j >= 0) {
                    const int k = j - qdiv(j, inv_ns) * ns;
                    if (ns > 1) {
#pragma unroll
                        for (int r = 1; r < RC; ++r) {
                            float2 t = tws[r * k * step];
                            if (SIGN > 0) t.y = -t.y;
                            v[bi][r] = cmul(v[bi][r], t);
                        }
                    }
                    if constexpr (RC == 2 || RC == 4) dft<RC, SIGN>(v[bi]);
                    else dft_odd<RC, SIGN>(v[bi]);
                    const int base = (j - k) * RC + k;
#pragma unroll
                    for (int r = 0; r < RC; ++r) a[rb[bi] * ld + base + r * ns] = v[bi][r];
                }
            }
        };
        switch (R) {
            case 4: run(std::integral_constant<int, 4>{}); break;
            case 2: run(std::integral_constant<int, 2>{}); break;
            case 3: run(std::integral_constant<int, 3>{}); break;
            case 5: run(std::integral_constant<int, 5>{}); break;
            default: run(std::integral_constant<int, 7>{}); break;
        }
        __syncthreads();
    }
}

// The twiddle table, copied into LDS when TWL (every thread's copy is
// ordered before the first pass by the barrier that follows the loads).
template <bool TWL>
__device__ __forceinline__ const float2* twiddle_table(float2* lds, const float2* __restrict__ twn, int n, int tid,
                                                       int nthr) {
    if constexpr (TWL) {
        for (int e = tid; e < n; e += nthr) lds[e] = twn[e];
        return lds;
    } else {
        (void)lds;
        return twn;
    }
}

// Column block (image, block kb of nkb) of hardware block L: in every group
// of 16 nkb consecutive blocks, the column blocks of two neighbouring images
// (channels c and c + 1 of the tiled spectrum share its 128-byte lines; in
// any layout they share the row spectrum's lines across column blocks) get
// indices equal mod 8 (the same XCD under round-robin dispatch) and
// consecutive dispatch slots, interleaved, so that the XCD's L2 fetches
// and writes back those lines once; a tail group keeps the plain order.
__device__ __forceinline__ void col_block(int64_t L, int nkb, int64_t nblocks, int64_t* img, int* kb) {
    const int64_t gsz = 16 * (int64_t)nkb;
    const int64_t g0 = L - L % gsz;
    if (g0 + gsz <= nblocks) {
        const int u = (int)(L - g0);
        const int sl = u / 8;                           // slot on the XCD: 0 .. 2 nkb - 1
        *img = g0 / nkb + 2 * (u % 8) + (sl & 1);
        *kb = sl >> 1;
        return;
    }
    *img = L / nkb;
    *kb = (int)(L % nkb);
}

// rows of length W = p.n (real) -> bins ky < my, two rows per complex
// transform (z = a + i b, A[k] = (Z[k] + conj Z[-k]) / 2, B[k] = (Z[k] - conj Z[-k]) / 2i).
// win: the rows are those of images of win.ph rows, and x holds only each
// image's top-left win.h x win.w corner (the rest reads as zero: the
// zero padding of a linear convolution).
template <int NE, bool TWL>
__global__ __launch_bounds__(kMrThreads) void k_rows_fwd_mr(const float* __restrict__ x, float2* __restrict__ y,
                                                            int64_t nrows, int my, int y_ld, float scale, MRPlan p,
                                                            const float2* __restrict__ twn, RowWindow win) {
    // rows longer than kLdsElems: one buffer (in-place passes) and the
    // block's two row offsets in a table of their own
    constexpr bool INP = NE > kLdsElems;
    __shared__ float2 buf[INP ? 1 : 2][NE];
    __shared__ float2 twl[TWL ? kMrTwLds : 1];
    __shared__ int64_t rtab[2];
    const int W = p.n;
    const int P = NE / W;
    const int tid = threadIdx.x;
    const float inv_w = 1.0f / (float)W;
    const float inv_my = 1.0f / (float)my;
    const double inv_ph = 1.0 / (double)win.ph;
    const float2* tws = twiddle_table<TWL>(twl, twn, W, tid, kMrThreads);
    const int64_t npairs = (nrows + 1) / 2;
    const int64_t pair0 = (int64_t)blockIdx.x * P;
    const int prows = (int)(npairs - pair0 < P ? npairs - pair0 : P);
    // Offset in x of each of the block's 2 prows rows, or -1 for a row of
    // zeros (padding rows, rows past the end), in the second buffer, which
    // the passes overwrite only later.  Row r is row q = r mod win.ph of
    // image r div win.ph (without a window, ph = h = 1: row r itself; row
    // indices fit 32 bits when a window is used: checked on the host); the
    // quotient is formed in double.
    int64_t* const srow = INP ? rtab : reinterpret_cast<int64_t*>(buf[INP ? 0 : 1]);
    for (int t = tid; t < 2 * prows; t += kMrThreads) {
        const int64_t r = 2 * pair0 + t;
        int64_t off = -1;
        if (r < nrows) {
            if (win.ph == 1) {
                off = r * win.w;
            } else {
                const uint32_t img = (uint32_t)(((double)(uint32_t)r + 0.5) * inv_ph);
                const int q = (int)((uint32_t)r - img * (uint32_t)win.ph);
                if (q < win.h) off = ((int64_t)img * win.h + q) * win.w;
            }
        }
        srow[t] = off;
    }
    __syncthreads();
    for (int e = tid; e < prows * W; e += kMrThreads) {
        const int pr = qdiv(e, inv_w);
        const int n = e - pr * W;
        const int64_t oa = srow[2 * pr], ob = srow[2 * pr + 1];
        const bool in = n < win.w;
        buf[0][e] = make_float2(in && oa >= 0 ? x[oa + n] : 0.0f, in && ob >= 0 ? x[ob + n] : 0.0f);
    }
    __syncthreads();
    const float2* res = buf[0];
    if constexpr (INP) fft_rows_mr_inplace<-1, NE>(buf[0], prows, W, p, tws, tid);
    else res = fft_rows_mr<-1>(buf[0], buf[INP ? 0 : 1], prows, W, p, tws, tid);
    // the block's 2 P rows of bins from a uniform base, 32-bit offsets
    // (2 P y_ld < 2^31: checked on the host)
    float2* const yb = y + 2 * pair0 * (int64_t)y_ld;
    const int64_t rows_left = nrows - 2 * pair0;
    const float hs = 0.5f * scale;
    for (int e = tid; e < prows * my; e += kMrThreads) {
        const int pr = qdiv(e, inv_my);
        const int k = e - pr * my;
        const float2 zk = res[pr * W + k];
        const float2 zm = res[pr * W + (k == 0 ? 0 : W - k)];
        const uint32_t o = (uint32_t)(2 * pr) * (uint32_t)y_ld + (uint32_t)k;
        yb[o] = make_float2(hs * (zk.x + zm.x), hs * (zk.y - zm.y));
        if (2 * pr + 1 < rows_left) yb[o + (uint32_t)y_ld] = make_float2(hs * (zk.y + zm.y), hs * (zm.x - zk.x));
    }
}

// Element (image img = b C + c, mode m) of a spectrum in layout `lay`.
__device__ __forceinline__ int64_t spec_at(const SpecLayout& lay, int64_t img, int m) {
    const int64_t b = img / lay.C;
    return b * lay.sb + (img - b * lay.C) * lay.sc + (int64_t)(m >> 3) * lay.st + (m & 7);
}

// R[nimg][H][my] -> xh (kept kx only, mode q my + ky, in layout `lay`),
// H = p.n
template <bool TWL>
__global__ __launch_bounds__(kMrThreads) void k_cols_fwd_mr(const float2* __restrict__ r, float2* __restrict__ xh,
                                                            SpecLayout lay, int mx, int my, int kb, int nkb,
                                                            float scale, MRPlan p, const float2* __restrict__ twn) {
    __shared__ float2 buf[2][kLdsElems];
    __shared__ float2 twl[TWL ? kMrTwLds : 1];
    const int H = p.n;
    const int tid = threadIdx.x;
    const float2* tws = twiddle_table<TWL>(twl, twn, H, tid, kMrThreads);
    int64_t img;
    int kbi;
    col_block(blockIdx.x, nkb, gridDim.x, &img, &kbi);
    const int ky0 = kbi * kb;
    const int ncol = min(kb, my - ky0);
    const float inv_ncol = 1.0f / (float)ncol;
    const int ld = H | 1;           // odd pitch: the column-wise accesses below hit distinct banks
    // the image's rows from a uniform base, 32-bit offsets (H my < 2^24)
    const float2* src = r + img * H * my + ky0;
    for (int e = tid; e < ncol * H; e += kMrThreads) {
        const int h = qdiv(e, inv_ncol);
        const int c = e - h * ncol;
        buf[0][c * ld + h] = src[(uint32_t)(h * my + c)];
    }
    __syncthreads();
    const float2* res = fft_rows_mr<-1>(buf[0], buf[1], ncol, ld, p, tws, tid);
    float2* dst = xh + spec_at(lay, img, 0);
    for (int e = tid; e < 2 * mx * ncol; e += kMrThreads) {
        const int q = qdiv(e, inv_ncol);
        const int c = e - q * ncol;
        const int kx = q < mx ? q : H - 2 * mx + q;
        const int m = q * my + ky0 + c;
        dst[(int64_t)(m >> 3) * lay.st + (m & 7)] = cscale(res[c * ld + kx], scale);
    }
}

// yh (mode q my + ky, in layout `lay`) -> zero-filled inverse along H ->
// R'[nimg][H][my]
template <bool TWL>
__global__ __launch_bounds__(kMrThreads) void k_cols_inv_mr(const float2* __restrict__ yh, float2* __restrict__ r,
                                                            SpecLayout lay, int mx, int my, int kb, int nkb, MRPlan p,
                                                            const float2* __restrict__ twn) {
    __shared__ float2 buf[2][kLdsElems];
    __shared__ float2 twl[TWL ? kMrTwLds : 1];
    const int H = p.n;
    const int tid = threadIdx.x;
    const float2* tws = twiddle_table<TWL>(twl, twn, H, tid, kMrThreads);
    int64_t img;
    int kbi;
    col_block(blockIdx.x, nkb, gridDim.x, &img, &kbi);
    const int ky0 = kbi * kb;
    const int ncol = min(kb, my - ky0);
    const float inv_ncol = 1.0f / (float)ncol;
    const float inv_h = 1.0f / (float)H;
    const int ld = H | 1;           // odd pitch: the column-wise accesses below hit distinct banks
    const float2* src = yh + spec_at(lay, img, 0);
    for (int e = tid; e < ncol * H; e += kMrThreads) {
        const int c = qdiv(e, inv_h);
        const int kx = e - c * H;
        if (kx >= mx && kx < H - mx) buf[0][c * ld + kx] = make_float2(0.0f, 0.0f);
    }
    for (int e = tid; e < 2 * mx * ncol; e += kMrThreads) {
        const int q = qdiv(e, inv_ncol);
        const int c = e - q * ncol;
        const int kx = q < mx ? q : H - 2 * mx + q;
        const int m = q * my + ky0 + c;
        buf[0][c * ld + kx] = src[(int64_t)(m >> 3) * lay.st + (m & 7)];
    }
    __syncthreads();
    const float2* res = fft_rows_mr<1>(buf[0], buf[1], ncol, ld, p, tws, tid);
    float2* dst = r + img * H * my + ky0;
    for (int e = tid; e < ncol * H; e += kMrThreads) {
        const int h = qdiv(e, inv_ncol);
        const int c = e - h * ncol;
        dst[(uint32_t)(h * my + c)] = res[c * ld + h];
    }
}

// R'[nrows][y_ld] (bins ky < my) -> C2R rows of length W = p.n, times scale
// (imaginary parts of the DC bin, and of the Nyquist bin when W is even,
// dropped); EPI: the fused output epilogue on every output.  win: only the
// window of rows [h0, h0 + h) x columns [w0, w0 + w) of each image of
// win.ph rows is written, packed (the crop of a linear convolution).
template <bool EPI, int NE, bool TWL>
__global__ __launch_bounds__(kMrThreads) void k_rows_inv_mr(const float2* __restrict__ y, float* __restrict__ out,
                                                            int64_t nrows, int my, int y_ld, float scale, MRPlan p,
                                                            const float2* __restrict__ twn, Epilogue epi,
                                                            RowWindow win) {
    constexpr bool INP = NE > kLdsElems;      // as in the forward: one buffer, in-place passes
    __shared__ float2 buf[INP ? 1 : 2][NE];
    __shared__ float2 twl[TWL ? kMrTwLds : 1];
    __shared__ int64_t rtab[2];
    const int W = p.n;
    const int P = NE / W;
    const int tid = threadIdx.x;
    const float inv_w = 1.0f / (float)W;
    const double inv_ph = 1.0 / (double)win.ph;
    const float2* tws = twiddle_table<TWL>(twl, twn, W, tid, kMrThreads);
    const int64_t npairs = (nrows + 1) / 2;
    const int64_t pair0 = (int64_t)blockIdx.x * P;
    const int prows = (int)(npairs - pair0 < P ? npairs - pair0 : P);
    // the block's 2 P rows of bins from a uniform base, 32-bit offsets
    // (2 P y_ld < 2^31: checked on the host)
    const float2* const ybase = y + 2 * pair0 * (int64_t)y_ld;
    const int64_t rows_left = nrows - 2 * pair0;
    for (int e = tid; e < prows * W; e += kMrThreads) {
        const int pr = qdiv(e, inv_w);
        const int k = e - pr * W;
        const int kk = (2 * k <= W) ? k : W - k;
        float2 z = make_float2(0.0f, 0.0f);
        if (kk < my) {
            const uint32_t o = (uint32_t)(2 * pr) * (uint32_t)y_ld + (uint32_t)kk;
            const float2 ya = ybase[o];
            const float2 yb = (2 * pr + 1 < rows_left) ? ybase[o + (uint32_t)y_ld] : make_float2(0.0f, 0.0f);
            if (kk == 0 || 2 * kk == W) z = make_float2(ya.x, yb.x);
            else if (k == kk) z = make_float2(ya.x - yb.y, ya.y + yb.x);
            else z = make_float2(ya.x + yb.y, yb.x - ya.y);
        }
        buf[0][e] = z;
    }
    __syncthreads();
    const float2* res = buf[0];
    if constexpr (INP) fft_rows_mr_inplace<1, NE>(buf[0], prows, W, p, tws, tid);
    else res = fft_rows_mr<1>(buf[0], buf[INP ? 0 : 1], prows, W, p, tws, tid);
    const bool crop = !(win.w == W && win.h == win.ph);
    // crop: offset in out of each of the block's 2 prows rows, or -1 for a
    // row outside the window; rows ra and ra + 1 may fall
    // in different images (the image index is the quotient by win.ph,
    // formed in double).  The table sits in the buffer the passes left free.
    int64_t* const drow = INP ? rtab : reinterpret_cast<int64_t*>(res == buf[0] ? buf[INP ? 0 : 1] : buf[0]);
    if (crop) {
        for (int t = tid; t < 2 * prows; t += kMrThreads) {
            const int64_t r = 2 * pair0 + t;
            int64_t off = -1;
            if (r < nrows) {
                const uint32_t img = (uint32_t)(((double)(uint32_t)r + 0.5) * inv_ph);
                const int q = (int)((uint32_t)r - img * (uint32_t)win.ph) - win.h0;
                if (q >= 0 && q < win.h) off = ((int64_t)img * win.h + q) * win.w;
            }
            drow[t] = off;
        }
        __syncthreads();
    }
    // uncropped output: the block's 2 P rows from a uniform base, 32-bit
    // offsets (2 P W <= 2 NE)
    float* const obase = out + 2 * pair0 * (int64_t)W;
    for (int e = tid; e < prows * W; e += kMrThreads) {
        const int pr = qdiv(e, inv_w);
        const int n = e - pr * W;
        const int64_t ra = 2 * (pair0 + pr);
        const uint32_t o = (uint32_t)(2 * pr * W + n);
        const float2 z = res[e];
        if (crop) {
            if (n < win.w0 || n >= win.w0 + win.w) continue;
            const int64_t oa = drow[2 * pr], ob = drow[2 * pr + 1];
            if (oa >= 0) nt_store(&out[oa + n - win.w0], z.x * scale);
            if (ob >= 0) nt_store(&out[ob + n - win.w0], z.y * scale);
            continue;
        }
        if constexpr (EPI) {
            const __amdgpu_buffer_rsrc_t rb =
                make_rsrc(epi.branch ? epi.branch + 2 * pair0 * W : nullptr,
                          epi.branch ? (uint32_t)((nrows - 2 * pair0 < 2 * P ? nrows - 2 * pair0 : 2 * P) * W * 4) : 0u);
            const uint32_t off = o * 4u;
            nt_store(&obase[o], epi_apply(epi, z.x * scale, epi_bias(epi, (uint32_t)ra), buffer_load_f1(rb, off, 0)));
            if (ra + 1 < nrows)
                nt_store(&obase[o + (uint32_t)W], epi_apply(epi, z.y * scale, epi_bias(epi, (uint32_t)(ra + 1)),
                                                            buffer_load_f1(rb, off + (uint32_t)W * 4u, 0)));
        } else {
            nt_store(&obase[o], z.x * scale);
            if (ra + 1 < nrows) nt_store(&obase[o + (uint32_t)W], z.y * scale);
        }
    }
}

// radix-4 passes first, then 2, 3, 5, 7
bool make_plan(int n, MRPlan* p, int nmax = kLdsElems) {
    if (n < 2 || n > nmax) return false;
    *p = MRPlan{};
    p->n = n;
    p->npass = 0;
    int m = n, ns = 1;
    for (int r : {4, 2, 3, 5, 7})
        while (m % r == 0) {
            if (p->npass == kMrMaxPasses) return false;
            const int k = p->npass++;
            p->r[k] = r;
            p->j[k] = n / r;
            p->ns[k] = ns;
            p->step[k] = n / (ns * r);
            p->inv_j[k] = (float)(1.0 / (double)(n / r));
            p->inv_ns[k] = (float)(1.0 / (double)ns);
            ns *= r;
            m /= r;
        }
    return m == 1;
}

// per (device, n) twiddle tables, built once and kept for the process
std::mutex g_tw_mutex;
std::map<std::pair<int, int>, float2*> g_tw;

// (a new table cannot be built while `s` is being captured: the allocation
// and the synchronous copy are refused with hipErrorStreamCaptureUnsupported)
hipError_t twiddles(int n, hipStream_t s, const float2** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_tw_mutex);
    auto it = g_tw.find({dev, n});
    if (it != g_tw.end()) {
        *out = it->second;
        return hipSuccess;
    }
    if (stream_capturing(s)) return hipErrorStreamCaptureUnsupported;
    std::vector<float2> host(n);
    for (int m = 0; m < n; ++m) {
        const double a = -2.0 * M_PI * (double)m / (double)n;
        host[m] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
    float2* d = nullptr;
    e = hipMalloc(&d, sizeof(float2) * n);
    if (e != hipSuccess) return e;
    e = hipMemcpy(d, host.data(), sizeof(float2) * n, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        return e;
    }
    g_tw[{dev, n}] = d;
    *out = d;
    return hipSuccess;
}

int64_t blocks_for(int64_t n) { return n < 1 ? 1 : n; }

}  // namespace

bool mixed_supported(int n) {
    MRPlan p;
    return make_plan(n, &p);
}

bool mixed_row_supported(int n) {
    MRPlan p;
    return make_plan(n, &p, kMrLongRow);
}

hipError_t launch_rows_fwd_mr(const float* x, float2* y, int64_t nrows, int W, int my, int y_ld, float scale,
                              hipStream_t s, const RowWindow* window) {
    MRPlan p;
    if (!make_plan(W, &p, kMrLongRow) || my > W / 2 + 1) return hipErrorInvalidValue;
    const float2* twn = nullptr;
    hipError_t e = twiddles(W, s, &twn);
    if (e != hipSuccess) return e;
    const bool lng = W > kLdsElems;
    const int P = (lng ? kMrLongRow : kLdsElems) / W;
    const int64_t nb = ((nrows + 1) / 2 + P - 1) / P;
    if (nb >= INT32_MAX || (int64_t)2 * P * y_ld >= INT32_MAX) return hipErrorInvalidValue;
    const RowWindow win = window ? *window : RowWindow{1, 1, W, 0, 0};
    if (win.ph < 1 || win.h < 1 || win.h > win.ph || win.w < 1 || win.w > W || nrows % win.ph ||
        (window && nrows >= INT32_MAX))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks_for(nb)), block(kMrThreads);
    if (lng)
        return launch_kernel(k_rows_fwd_mr<kMrLongRow, false>, grid, block, 0, s, x, y, nrows, my, y_ld, scale, p, twn,
                             win);
    if (W <= kMrTwLds)
        return launch_kernel(k_rows_fwd_mr<kLdsElems, true>, grid, block, 0, s, x, y, nrows, my, y_ld, scale, p, twn,
                             win);
    return launch_kernel(k_rows_fwd_mr<kLdsElems, false>, grid, block, 0, s, x, y, nrows, my, y_ld, scale, p, twn, win);
}

hipError_t launch_cols_fwd_mr(const float2* r, float2* xh, int64_t nimg, int H, int mx, int my, float scale,
                              hipStream_t s, const SpecLayout* layout) {
    MRPlan p;
    if (!make_plan(H, &p) || 2 * mx > H) return hipErrorInvalidValue;
    const float2* twn = nullptr;
    hipError_t e = twiddles(H, s, &twn);
    if (e != hipSuccess) return e;
    const int cap = kLdsElems / (H | 1);       // columns at the kernel's odd pitch
    if (cap < 1) return hipErrorInvalidValue;
    const int kb = cap < my ? cap : my;
    const int nkb = (my + kb - 1) / kb;
    const int64_t nb = nimg * nkb;
    if (nb >= INT32_MAX) return hipErrorInvalidValue;
    // default: image after image, 2 mx my modes each
    const SpecLayout lay = layout ? *layout : SpecLayout{(int64_t)2 * mx * my, 0, 8, 1};
    if (lay.C < 1 || lay.st < 8) return hipErrorInvalidValue;
    if (H <= kMrTwLds)
        return launch_kernel(k_cols_fwd_mr<true>, dim3((unsigned)nb), dim3(kMrThreads), 0, s, r, xh, lay, mx, my,
                             kb, nkb, scale, p, twn);
    return launch_kernel(k_cols_fwd_mr<false>, dim3((unsigned)nb), dim3(kMrThreads), 0, s, r, xh, lay, mx, my, kb,
                         nkb, scale, p, twn);
}

hipError_t launch_cols_inv_mr(const float2* yh, float2* r, int64_t nimg, int H, int mx, int my, hipStream_t s,
                              const SpecLayout* layout) {
    MRPlan p;
    if (!make_plan(H, &p) || 2 * mx > H) return hipErrorInvalidValue;
    const float2* twn = nullptr;
    hipError_t e = twiddles(H, s, &twn);
    if (e != hipSuccess) return e;
    const int cap = kLdsElems / (H | 1);       // columns at the kernel's odd pitch
    if (cap < 1) return hipErrorInvalidValue;
    const int kb = cap < my ? cap : my;
    const int nkb = (my + kb - 1) / kb;
    const int64_t nb = nimg * nkb;
    if (nb >= INT32_MAX) return hipErrorInvalidValue;
    // default: image after image, 2 mx my modes each
    const SpecLayout lay = layout ? *layout : SpecLayout{(int64_t)2 * mx * my, 0, 8, 1};
    if (lay.C < 1 || lay.st < 8) return hipErrorInvalidValue;
    if (H <= kMrTwLds)
        return launch_kernel(k_cols_inv_mr<true>, dim3((unsigned)nb), dim3(kMrThreads), 0, s, yh, r, lay, mx, my,
                             kb, nkb, p, twn);
    return launch_kernel(k_cols_inv_mr<false>, dim3((unsigned)nb), dim3(kMrThreads), 0, s, yh, r, lay, mx, my, kb,
                         nkb, p, twn);
}

hipError_t launch_rows_inv_mr(const float2* y, float* out, int64_t nrows, int W, int my, int y_ld, float scale,
                              hipStream_t s, const Epilogue& epi, const RowWindow* window) {
    MRPlan p;
    if (!make_plan(W, &p, kMrLongRow) || my > W / 2 + 1) return hipErrorInvalidValue;
    const bool lng = W > kLdsElems;
    if (lng && epi.on) return hipErrorInvalidValue;      // the long rows serve the linear convolution only
    const float2* twn = nullptr;
    hipError_t e = twiddles(W, s, &twn);
    if (e != hipSuccess) return e;
    const int P = (lng ? kMrLongRow : kLdsElems) / W;
    const int64_t nb = ((nrows + 1) / 2 + P - 1) / P;
    if (nb >= INT32_MAX || (int64_t)2 * P * y_ld >= INT32_MAX) return hipErrorInvalidValue;
    const RowWindow win = window ? *window : RowWindow{1, 1, W, 0, 0};
    if (win.ph < 1 || win.h < 1 || win.h0 < 0 || win.h0 + win.h > win.ph || win.w < 1 || win.w0 < 0 ||
        win.w0 + win.w > W || nrows % win.ph || (window && (epi.on || nrows >= INT32_MAX)))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks_for(nb)), block(kMrThreads);
    if (lng)
        return launch_kernel(k_rows_inv_mr<false, kMrLongRow, false>, grid, block, 0, s, y, out, nrows, my, y_ld, scale,
                             p, twn, epi, win);
    if (W <= kMrTwLds) {
        if (epi.on)
            return launch_kernel(k_rows_inv_mr<true, kLdsElems, true>, grid, block, 0, s, y, out, nrows, my, y_ld, scale,
                                 p, twn, epi, win);
        return launch_kernel(k_rows_inv_mr<false, kLdsElems, true>, grid, block, 0, s, y, out, nrows, my, y_ld, scale, p,
                             twn, epi, win);
    }
    if (epi.on)
        return launch_kernel(k_rows_inv_mr<true, kLdsElems, false>, grid, block, 0, s, y, out, nrows, my, y_ld, scale, p,
                             twn, epi, win);
    return launch_kernel(k_rows_inv_mr<false, kLdsElems, false>, grid, block, 0, s, y, out, nrows, my, y_ld, scale, p,
                         twn, epi, win);
}

}  // namespace fno
