// Forward transform with register-resident rows, for 64x64 .. 128x128 grids.
//
// Row pass: one thread per real row.  The row is taken as W/2 complex
// samples z[n] = x[2n] + i x[2n+1] and the whole W/2-point DFT runs in the
// thread's registers, with no exchange and no barrier.  The real row's half
// spectrum follows from the even / odd split (FFT blog, section 2.2: R2C
// keeps the N/2+1 half spectrum):
//   a = Z[k] + conj Z[W/2-k],  b = Z[k] - conj Z[W/2-k],
//   X[k] = a / 2 + W_W^k (-i / 2) b,   k < my,
// with the ortho factor (HW)^-1/2 folded into those constants.
// Column pass (TurboFNO blog, sections 2.1-2.2: the second 1D transform of
// the 2D one, only the kept kx written): the X plane sits in LDS; batches of
// KB columns are split H = R1 * R2 (R1 points per thread: an R1-point DFT
// in registers, the twiddle W_H^{t k1}, a hand-over through LDS, R2-point
// DFTs across threads) and only kx in [0,mx) u [H-mx,H) are stored.
//
// Data movement: the rows arrive through coalesced loads (8 lanes per
// 128-byte run) and a wave-private LDS transpose hands each lane its own row.
// The transpose stage, the X plane and the hand-over buffers share one LDS
// region (about 35 KiB at 128 x 128), so four workgroups of two waves fit on
// a CU: two waves per SIMD, one doing VALU work while the other waits on LDS
// or HBM.  The grid is persistent (as many workgroups as fit), each walking
// images in XCD-paired order; the output goes through buffer stores whose
// hardware range check drops the outputs of dropped modes.
#include <cstdint>

#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

template <int N> struct ColSplit;
template <> struct ColSplit<64>  { static constexpr int R1 = 8,  R2 = 8; };
template <> struct ColSplit<128> { static constexpr int R1 = 16, R2 = 8; };

// Base of image img = b * C + c in a mode-addressed spectrum (complex elements).
struct ImageBase {
    int64_t sb, sc;
    int C;
    __device__ __forceinline__ int64_t operator()(int64_t img) const {
        const uint32_t i32 = (uint32_t)img;
        const uint32_t b = i32 / (uint32_t)C;
        const uint32_t c = i32 - b * (uint32_t)C;
        return (int64_t)b * sb + (int64_t)c * sc;
    }
};

// 2^(-e/2)
constexpr double inv_sqrt_pow2(int e) {
    double v = 1.0;
    for (int i = 0; i < e / 2; ++i) v *= 0.5;
    return (e & 1) ? v * 0.70710678118654752440 : v;
}

template <int LOG2H, int LOG2W, int MYMAX>
struct RowPlan {
    static constexpr int H = 1 << LOG2H;
    static constexpr int W = 1 << LOG2W;
    static constexpr int NZ = W / 2;                // complex samples per row
    static constexpr int NT = H;                    // threads: one per row
    static constexpr int F4 = W / 4;                // float4 per row
    static constexpr int NCK = F4 / 8;              // 128-byte runs per row
    static constexpr int R1 = ColSplit<H>::R1;
    static constexpr int R2 = ColSplit<H>::R2;
    static constexpr int NJ = R1 / R2;              // second-stage DFTs per thread
    static constexpr int KB = NT / R2;              // columns per batch
    static constexpr int NB = MYMAX / KB;           // batches
    static constexpr int PS = MYMAX + 1;            // plane row stride (odd)
    static constexpr int XS = R1 + 1;               // hand-over slot stride (odd)
    static constexpr int GS = (R2 * XS) | 1;        // hand-over column stride (odd)
    static constexpr int SS = 36;                   // transpose stage row stride (floats)
    static constexpr int PLANE = H * PS;            // complex elements
    static constexpr int XBUF = KB * GS;
    static constexpr int XBUFS = NB * XBUF;         // one hand-over buffer per batch
    static constexpr int STAGE = NT * SS / 2;
    static constexpr int XREG = XBUFS > STAGE ? XBUFS : STAGE;
    // the stage, the plane and the hand-over buffers share one region,
    // behind a table of the column twiddles W_H^j
    static constexpr int REGION = H + (PLANE > XREG ? PLANE : XREG);
    static_assert(MYMAX % KB == 0 && MYMAX <= NZ, "column batches");
    static_assert(R1 % R2 == 0, "column split");
    static size_t lds_bytes() { return sizeof(float2) * (size_t)REGION; }
};

// MXK > 0: the kept kx count per side is MXK, a multiple of R1, known when the
// kernel is compiled.  Column-stage index k2 then covers kx in
// [R1 k2, R1 k2 + R1), a block that is either wholly kept or wholly dropped,
// so the forward need not form (and the inverse need not read) the dropped
// blocks.  MXK = 0: mx is read at run time and every block is formed.
template <int H, int R1, int MXK>
__device__ constexpr bool block_kept(int k2) {
    return MXK == 0 || R1 * k2 + R1 <= MXK || R1 * k2 >= H - MXK;
}

// Bin K of the scaled half spectrum of a real row of length W from its packed
// transform Z (NZ = W/2 points), s = 2^(-LOG2HW/2):
//   s X[K] = (s/2) a + c b,   c = (s/2) (-i) W_W^K = (s/2) (-sin, -cos)(2 pi K / W).
template <int W, int K, int NZ, int LOG2HW>
__device__ __forceinline__ float2 half_bin_scaled(const float2 (&z)[NZ]) {
    constexpr double hs = 0.5 * inv_sqrt_pow2(LOG2HW);
    constexpr float h = (float)hs;
    const float2 zk = z[K % NZ];
    const float2 zm = z[(NZ - K % NZ) % NZ];
    const float ax = zk.x + zm.x, ay = zk.y - zm.y;
    const float bx = zk.x - zm.x, by = zk.y + zm.y;
    constexpr double sn = exact_sin(K, W), cs = exact_cos(K, W);
    float tx, ty;
    if constexpr (sn == 0.0) {          // c = (0, -h cos)
        constexpr float ci = (float)(-hs * cs);
        tx = -by * ci;
        ty = bx * ci;
    } else if constexpr (cs == 0.0) {   // c = (-h sin, 0)
        constexpr float cr = (float)(-hs * sn);
        tx = bx * cr;
        ty = by * cr;
    } else {
        // expanded over zk and zm, the constants h +- cr formed in double:
        // four fused multiply-adds per part instead of the pre-sums
        constexpr double crd = -hs * sn;
        constexpr float p = (float)(hs + crd), m = (float)(hs - crd), ci = (float)(-hs * cs);
        (void)ax, (void)ay, (void)bx, (void)by;
        return make_float2(fmaf(p, zk.x, fmaf(m, zm.x, fmaf(-ci, zk.y, -ci * zm.y))),
                           fmaf(p, zk.y, fmaf(-m, zm.y, fmaf(ci, zk.x, -ci * zm.x))));
    }
    return make_float2(fmaf(h, ax, tx), fmaf(h, ay, ty));
}

// DIAG: the diagonal global filter folded into the store: every kept mode m
// of image b C + c is multiplied by mask[c][m] (the mask transposed
// channel-major, so that a wave's lanes, over consecutive ky, read
// consecutive entries) on its way out.
template <int LOG2H, int LOG2W, int MYMAX, bool DIAG, int MXK>
__global__ __launch_bounds__(1 << LOG2H) __attribute__((amdgpu_waves_per_eu(2))) void k_fwd2d_rows(const float* __restrict__ x, float2* __restrict__ xh,
                                                           ImageBase ib, int st, int64_t nimg, int mx, int my,
                                                           const float2* __restrict__ tw,
                                                           const float2* __restrict__ mask) {
    using S = RowPlan<LOG2H, LOG2W, MYMAX>;
    constexpr int H = S::H, W = S::W, NZ = S::NZ, F4 = S::F4, R1 = S::R1, R2 = S::R2, KB = S::KB, NB = S::NB,
                  NJ = S::NJ;
    extern __shared__ float2 smem[];
    float2* const twH = smem;                   // W_H^j, j < H
    float2* const plane = smem + H;             // [H][PS]: scaled X of every row
    float2* const xreg = smem + H;              // transpose stage / hand-over buffers (same region)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int t = tid / KB;                     // column pass: slot t of column cl
    const int cl = tid % KB;
    twH[tid] = tw[tid * (kNMax / H)];           // NT == H: one entry per thread

    // Per-thread constants for the stores: q * my for every output (k1 = t +
    // R2 jj, k2) of the last column stage, where q is the row of kx = k1 +
    // R1 k2 in the truncated spectrum (-1: kx is not kept).
    int qm[NJ][R2];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int k2 = 0; k2 < R2; ++k2) {
            const int kx = t + R2 * jj + R1 * k2;
            const int q = kx < mx ? kx : (kx >= H - mx ? kx - (H - 2 * mx) : -1);
            qm[jj][k2] = q < 0 ? -1 : q * my;
        }
    const uint32_t out_bytes = (uint32_t)((((2 * mx * my) - 1) >> 3) * st + 8) * 8u;
    const uint32_t st8 = (uint32_t)(st - 8);

    // Coalesced row loads: load i = (run c, group ii) of lane l reads float4
    // 8c + (l & 7) of row 8 ii + (l >> 3) of the wave's 64 rows.
    uint32_t loff[8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) loff[ii] = (uint32_t)(((tid & ~63) + 8 * ii + (lane >> 3)) * F4 + (lane & 7)) * 16u;
    float2 ld[2 * F4];
    auto issue = [&](int64_t img) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(x + img * (int64_t)(H * W), (uint32_t)(H * W * 4));
        static_for<0, F4>([&](auto i) {
            constexpr int c = i / 8, ii = i % 8;
            const float4 v = buffer_load_f4(r, loff[ii] + 128 * c, 0);
            ld[2 * i] = make_float2(v.x, v.y);
            ld[2 * i + 1] = make_float2(v.z, v.w);
        });
    };

    const int64_t G = gridDim.x;
    int64_t L = blockIdx.x;
    for (; L < nimg; L += G) {
        const int64_t img = paired_image(L, nimg);
        issue(img);
        lds_barrier();                          // the previous image is out of the shared region

        // ---- hand the loaded rows over: lane l gets row l of its wave ------
        float2 z[NZ];
        {
            float* stage = reinterpret_cast<float*>(xreg) + (tid >> 6) * 64 * S::SS;
            static_for<0, S::NCK>([&](auto c) {
                static_for<0, 8>([&](auto ii) {
                    constexpr int i = c * 8 + ii;
                    *reinterpret_cast<float4*>(stage + (8 * ii + (lane >> 3)) * S::SS + 4 * (lane & 7)) =
                        make_float4(ld[2 * i].x, ld[2 * i].y, ld[2 * i + 1].x, ld[2 * i + 1].y);
                });
                wave_lds_sync();
                static_for<0, 8>([&](auto q) {
                    const float4 v = *reinterpret_cast<const float4*>(stage + lane * S::SS + 4 * q);
                    z[2 * (8 * c + q)] = make_float2(v.x, v.y);
                    z[2 * (8 * c + q) + 1] = make_float2(v.z, v.w);
                });
                wave_lds_sync();
            });
        }
        lds_barrier();                          // every wave is out of the stage before the plane is written

        // ---- row tid: packed W/2-point DFT, scaled half spectrum -> plane --
        dft<NZ, -1>(z);
        static_for<0, MYMAX>([&](auto k) {
            plane[tid * S::PS + k] = half_bin_scaled<W, k, NZ, LOG2H + LOG2W>(z);
        });
        lds_barrier();

        // ---- columns: every batch's first stage, one hand-over, last stage -
        float2 v[NB][R1];
        static_for<0, NB>([&](auto bt) {
#pragma unroll
            for (int m = 0; m < R1; ++m) v[bt][m] = plane[(t + R2 * m) * S::PS + bt * KB + cl];
        });
        lds_barrier();                          // the plane is read before the hand-over overwrites it
        static_for<0, NB>([&](auto bt) {
            dft<R1, -1>(v[bt]);
#pragma unroll
            for (int k1 = 1; k1 < R1; ++k1) v[bt][k1] = cmul(v[bt][k1], twH[(t * k1) & (H - 1)]);
            float2* const xb = xreg + bt * S::XBUF + cl * S::GS + t * S::XS;
#pragma unroll
            for (int k1 = 0; k1 < R1; ++k1) xb[k1] = v[bt][k1];
        });
        lds_barrier();
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(xh + ib(img), out_bytes);
        // filter: image b C + c reads row c of the transposed mask; dropped
        // modes read zero through the range check
        __amdgpu_buffer_rsrc_t rmask = ro;
        if constexpr (DIAG) {
            const uint32_t c = (uint32_t)img % (uint32_t)ib.C;
            rmask = make_rsrc(mask + (int64_t)c * (2 * mx * my), (uint32_t)(2 * mx * my) * 8u);
        }
        static_for<0, NB>([&](auto bt) {
            const float2* const xb = xreg + bt * S::XBUF + cl * S::GS;
            const int ky = bt * KB + cl;
            const bool kyok = ky < my;
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const int k1 = t + R2 * jj;
                float2 u[R2];
                float2 mv[DIAG ? R2 : 1];
                if constexpr (DIAG) {
                    static_for<0, R2>([&](auto k2) {
                        if constexpr (block_kept<H, R1, MXK>(k2)) {
                            const int q = qm[jj][k2];
                            mv[k2] = buffer_load_f2(rmask, (q < 0 || !kyok) ? kBufferSkip : (uint32_t)(q + ky) * 8u, 0);
                        }
                    });
                }
#pragma unroll
                for (int tt = 0; tt < R2; ++tt) u[tt] = xb[tt * S::XS + k1];
                dft<R2, -1>(u);
                static_for<0, R2>([&](auto k2) {
                    if constexpr (block_kept<H, R1, MXK>(k2)) {
                        // mode m = q my + ky at (m >> 3) st + (m & 7) = m + (m >> 3)(st - 8)
                        const int q = qm[jj][k2];
                        const uint32_t m = (uint32_t)(q + ky);
                        const uint32_t off = (q < 0 || !kyok) ? kBufferSkip : (m + (m >> 3) * st8) * 8u;
                        float2 val = u[k2];
                        if constexpr (DIAG) val = cmul(val, mv[k2]);
                        buffer_store_f2(val, ro, off, 0);
                    }
                });
            }
        });
    }
}

// Bin k of the packed inverse row spectrum, for the C2R of a real row of
// length W whose half spectrum X is zero from MYMAX on (FFT blog, section
// 2.2: C2R from the N/2+1 half spectrum, imaginary part of the DC bin
// ignored).  With x[2n] + i x[2n+1] = IDFT_{W/2}(Z)[n]:
//   Z[k] = s (X[k] + conj X[W/2-k]) + c (X[k] - conj X[W/2-k]),
//   c = s i W_W^{-k} = s (-sin, cos)(2 pi k / W),   s = 2^(-LOG2HW/2).
template <int W, int K, int MYMAX, int LOG2HW>
__device__ __forceinline__ float2 packed_c2r_bin(const float2 (&X)[MYMAX]) {
    constexpr int NZ = W / 2;
    constexpr double s = inv_sqrt_pow2(LOG2HW);
    constexpr double sn = exact_sin(K, W), cs = exact_cos(K, W);
    constexpr bool has_k = K < MYMAX;
    constexpr bool has_m = K > 0 && NZ - K < MYMAX;
    if constexpr (K == 0) {
        // X[0] real, X[W/2] = 0: Z[0] = s Re X[0] (1 + i)
        const float v = (float)s * X[0].x;
        return make_float2(v, v);
    } else if constexpr (has_k && has_m) {
        const float2 xk = X[K], xm = X[has_m ? NZ - K : 0];
        const float ax = xk.x + xm.x, ay = xk.y - xm.y;
        const float bx = xk.x - xm.x, by = xk.y + xm.y;
        constexpr float cr = (float)(-s * sn), ci = (float)(s * cs), sf = (float)s;
        return make_float2(fmaf(sf, ax, fmaf(bx, cr, -by * ci)), fmaf(sf, ay, fmaf(bx, ci, by * cr)));
    } else if constexpr (has_k) {
        // Z = (s + c) X[k]
        constexpr float pr = (float)(s - s * sn), pi = (float)(s * cs);
        const float2 xk = X[has_k ? K : 0];
        return make_float2(fmaf(xk.x, pr, -xk.y * pi), fmaf(xk.x, pi, xk.y * pr));
    } else if constexpr (has_m) {
        // Z = (s - c) conj X[W/2-k]
        constexpr float pr = (float)(s + s * sn), pi = (float)(-s * cs);
        const float2 xm = X[has_m ? NZ - K : 0];
        return make_float2(fmaf(xm.x, pr, xm.y * pi), fmaf(xm.x, pi, -xm.y * pr));
    } else {
        return make_float2(0.0f, 0.0f);
    }
}

// Inverse of k_fwd2d_rows: truncated spectrum (kept kx only, ky < my, the
// rest zero) -> real image, scaled by (HW)^-1/2.  Column pass first
// (kx = k1 + R1 k2 -> h = t + R2 m: R2-point inverse DFTs over k2 read straight
// from the spectrum, the hand-over, the twiddle conj W_H^{t k1}, R1-point
// inverse DFTs over k1), its rows in the LDS plane; then one thread per row
// builds the packed spectrum Z, runs the W/2-point inverse DFT in registers
// and hands its row out through the stage to coalesced buffer stores.  EPI:
// the fused output epilogue (bias, GELU, second branch) is applied to each
// float4 between the stage and the store; a chunk's branch float4s are
// loaded only once that chunk of the rows has left the registers for the
// stage (the row registers are the kernel's peak).
template <int LOG2H, int LOG2W, int MYMAX, bool EPI, int MXK>
__global__ __launch_bounds__(1 << LOG2H) __attribute__((amdgpu_waves_per_eu(2))) void k_inv2d_rows(
    const float2* __restrict__ yh, float* __restrict__ out, ImageBase ib, int st, int64_t nimg, int mx, int my,
    const float2* __restrict__ tw, Epilogue epi) {
    using S = RowPlan<LOG2H, LOG2W, MYMAX>;
    constexpr int H = S::H, W = S::W, NZ = S::NZ, F4 = S::F4, R1 = S::R1, R2 = S::R2, KB = S::KB, NB = S::NB,
                  NJ = S::NJ;
    extern __shared__ float2 smem[];
    float2* const twH = smem;                   // W_H^j, j < H
    float2* const plane = smem + H;             // [H][PS]: column-inverted spectrum, one row per thread
    float2* const xreg = smem + H;              // hand-over buffers / output stage (same region)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int t = tid / KB;                     // column pass: slot t of column cl
    const int cl = tid % KB;
    twH[tid] = tw[tid * (kNMax / H)];           // NT == H: one entry per thread

    // q * my for every input (k1 = t + R2 jj, k2) of the first column stage
    // (q: row of kx = k1 + R1 k2 in the truncated spectrum, -1: not kept)
    int qm[NJ][R2];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
        for (int k2 = 0; k2 < R2; ++k2) {
            const int kx = t + R2 * jj + R1 * k2;
            const int q = kx < mx ? kx : (kx >= H - mx ? kx - (H - 2 * mx) : -1);
            qm[jj][k2] = q < 0 ? -1 : q * my;
        }
    const uint32_t in_bytes = (uint32_t)((((2 * mx * my) - 1) >> 3) * st + 8) * 8u;
    const uint32_t st8 = (uint32_t)(st - 8);
    // coalesced output: store (run c, group ii) of lane l writes float4
    // 8c + (l & 7) of row 8 ii + (l >> 3) of the wave's 64 rows
    uint32_t soffs[8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
        soffs[ii] = (uint32_t)(((tid & ~63) + 8 * ii + (lane >> 3)) * F4 + (lane & 7)) * 16u;

    const int64_t G = gridDim.x;
    for (int64_t L = blockIdx.x; L < nimg; L += G) {
        const int64_t img = paired_image(L, nimg);
        lds_barrier();                          // the previous image is out of the shared region

        // ---- columns, first stage: R2-point inverse DFTs over k2 ----------
        // Dropped modes read as zero through the buffer range check.
        const __amdgpu_buffer_rsrc_t ri = make_rsrc(yh + ib(img), in_bytes);
        float2 g[NB][NJ][R2];
        static_for<0, NB>([&](auto bt) {
            const int ky = bt * KB + cl;
            const bool kyok = ky < my;
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj)
                static_for<0, R2>([&](auto k2) {
                    if constexpr (block_kept<H, R1, MXK>(k2)) {
                        const int q = qm[jj][k2];
                        const uint32_t m = (uint32_t)(q + ky);
                        const uint32_t off = (q < 0 || !kyok) ? kBufferSkip : (m + (m >> 3) * st8) * 8u;
                        g[bt][jj][k2] = buffer_load_f2(ri, off, 0);
                    } else {
                        g[bt][jj][k2] = make_float2(0.0f, 0.0f);
                    }
                });
        });
        static_for<0, NB>([&](auto bt) {
            float2* const xb = xreg + bt * S::XBUF + cl * S::GS;
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                dft<R2, 1>(g[bt][jj]);
#pragma unroll
                for (int tt = 0; tt < R2; ++tt) xb[tt * S::XS + t + R2 * jj] = g[bt][jj][tt];
            }
        });
        lds_barrier();

        // ---- columns, second stage: twiddle, R1-point inverse DFTs over k1 -
        float2 v[NB][R1];
        static_for<0, NB>([&](auto bt) {
            const float2* const xb = xreg + bt * S::XBUF + cl * S::GS + t * S::XS;
#pragma unroll
            for (int k1 = 0; k1 < R1; ++k1) v[bt][k1] = xb[k1];
        });
        lds_barrier();                          // the hand-over is read before the plane overwrites it
        static_for<0, NB>([&](auto bt) {
#pragma unroll
            for (int k1 = 1; k1 < R1; ++k1) {
                const float2 w = twH[(t * k1) & (H - 1)];
                v[bt][k1] = cmul(v[bt][k1], make_float2(w.x, -w.y));
            }
            dft<R1, 1>(v[bt]);
#pragma unroll
            for (int m = 0; m < R1; ++m) plane[(t + R2 * m) * S::PS + bt * KB + cl] = v[bt][m];
        });
        lds_barrier();

        // ---- row tid: packed C2R in registers ------------------------------
        float2 z[NZ];
        {
            float2 X[MYMAX];
#pragma unroll
            for (int k = 0; k < MYMAX; ++k) X[k] = plane[tid * S::PS + k];
            static_for<0, NZ>([&](auto k) { z[k] = packed_c2r_bin<W, k, MYMAX, LOG2H + LOG2W>(X); });
        }
        dft<NZ, 1>(z);
        lds_barrier();                          // every row is out of the plane before the stage is written

        // ---- hand the row out: coalesced stores through the stage ---------
        {
            const __amdgpu_buffer_rsrc_t ro = make_rsrc(out + img * (int64_t)(H * W), (uint32_t)(H * W * 4));
            float* stage = reinterpret_cast<float*>(xreg) + (tid >> 6) * 64 * S::SS;
            // epilogue: the image's bias, its branch image (a null branch gets
            // an empty range: its loads read zero)
            float bias = 0.0f;
            __amdgpu_buffer_rsrc_t rb = ro;
            if constexpr (EPI) {
                bias = epi_bias(epi, (uint32_t)img);
                rb = make_rsrc(epi.branch ? epi.branch + img * (int64_t)(H * W) : nullptr,
                               epi.branch ? (uint32_t)(H * W * 4) : 0u);
            }
            // chunk c: float4 8c .. 8c+7 of every row of the wave (128-byte
            // column slabs of the image)
            auto emit = [&](auto c) __attribute__((always_inline)) {
                static_for<0, 8>([&](auto q) {
                    *reinterpret_cast<float4*>(stage + lane * S::SS + 4 * q) =
                        make_float4(z[2 * (8 * c + q)].x, z[2 * (8 * c + q)].y, z[2 * (8 * c + q) + 1].x,
                                    z[2 * (8 * c + q) + 1].y);
                });
                float4 br[EPI ? 8 : 1];
                if constexpr (EPI) {
                    __builtin_amdgcn_sched_barrier(0);      // the chunk's rows are in the stage first
                    static_for<0, 8>([&](auto ii) { br[ii] = buffer_load_f4(rb, soffs[ii] + 128 * c, 0); });
                }
                wave_lds_sync();
                static_for<0, 8>([&](auto ii) {
                    float4 o =
                        *reinterpret_cast<const float4*>(stage + (8 * ii + (lane >> 3)) * S::SS + 4 * (lane & 7));
                    if constexpr (EPI) {
                        o = make_float4(epi_apply(epi, o.x, bias, br[ii].x), epi_apply(epi, o.y, bias, br[ii].y),
                                        epi_apply(epi, o.z, bias, br[ii].z), epi_apply(epi, o.w, bias, br[ii].w));
                    }
                    buffer_store_f4_nt(o, ro, soffs[ii] + 128 * c, 0);
                });
                wave_lds_sync();
            };
            // Each workgroup starts at its own slab, so that the workgroups
            // (which run nearly in step) do not all write the same slab of
            // their images at once (measured at 128x128: 33.9-34.2 -> 33.0 us).
            const int rot = (int)(blockIdx.x % S::NCK);
            static_for<0, S::NCK>([&](auto r) {
                if (rot == r)
                    static_for<0, S::NCK>([&](auto i) { emit(std::integral_constant<int, (i + r) % S::NCK>{}); });
            });
        }
    }
}

// Launches kernel k on a persistent grid: as many workgroups as fit on the
// device (from the occupancy of k with `lds` bytes), in whole groups of 16
// for the XCD pairing, never more than there are images.
template <typename K, typename... A>
hipError_t launch_persistent(K k, int nt, size_t lds, int64_t nimg, hipStream_t s, A... args) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, nt, lds);
    if (e != hipSuccess) return e;
    int64_t g = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    g = g >= 16 ? (g / 16) * 16 : g;
    if (g > nimg) g = nimg;
    return launch_kernel(k, dim3((unsigned)g), dim3(nt), lds, s, args...);
}

// The 128 x 128 grid with 32 kept kx per side (the 128x128 PDE workload's
// shape) gets kernels compiled for that mx; every other shape reads mx at run
// time.
template <int LH, int LW>
constexpr bool has_mx32() { return LH == 7; }

template <int LH, int LW, int MYM>
hipError_t launch_fwd_one(const float* x, float2* xh, const ImageBase& ib, int st, int64_t nimg, int mx, int my,
                          const float2* tw, hipStream_t s, const float2* mask) {
    using P = RowPlan<LH, LW, MYM>;
    if constexpr (has_mx32<LH, LW>() && MYM == 32) {
        if (mx == 32 && !mask)
            return launch_persistent(k_fwd2d_rows<LH, LW, MYM, false, 32>, P::NT, P::lds_bytes(), nimg, s, x, xh, ib,
                                     st, nimg, mx, my, tw, mask);
    }
    if (mask)
        return launch_persistent(k_fwd2d_rows<LH, LW, MYM, true, 0>, P::NT, P::lds_bytes(), nimg, s, x, xh, ib, st,
                                 nimg, mx, my, tw, mask);
    return launch_persistent(k_fwd2d_rows<LH, LW, MYM, false, 0>, P::NT, P::lds_bytes(), nimg, s, x, xh, ib, st, nimg,
                             mx, my, tw, mask);
}

template <int LH, int LW, int MYM>
hipError_t launch_inv_one(const float2* yh, float* out, const ImageBase& ib, int st, int64_t nimg, int mx, int my,
                          const float2* tw, hipStream_t s, const Epilogue& epi) {
    using P = RowPlan<LH, LW, MYM>;
    if constexpr (has_mx32<LH, LW>() && MYM == 32) {
        if (mx == 32 && !epi.on)
            return launch_persistent(k_inv2d_rows<LH, LW, MYM, false, 32>, P::NT, P::lds_bytes(), nimg, s, yh, out,
                                     ib, st, nimg, mx, my, tw, epi);
    }
    if (epi.on)
        return launch_persistent(k_inv2d_rows<LH, LW, MYM, true, 0>, P::NT, P::lds_bytes(), nimg, s, yh, out, ib, st,
                                 nimg, mx, my, tw, epi);
    return launch_persistent(k_inv2d_rows<LH, LW, MYM, false, 0>, P::NT, P::lds_bytes(), nimg, s, yh, out, ib, st,
                             nimg, mx, my, tw, epi);
}

ImageBase image_base(const SpecLayout& lay) {
    ImageBase ib;
    ib.sb = lay.sb;
    ib.sc = lay.sc;
    ib.C = lay.C;
    return ib;
}

}  // namespace

bool rowreg2d_supported(int log2H, int log2W, int mx, int my, const SpecLayout& lay) {
    // byte offsets inside one image's spectrum stay below kBufferSkip
    const int64_t tiles = ((int64_t)2 * mx * my + 7) / 8;
    return (log2H == 6 || log2H == 7) && (log2W == 6 || log2W == 7) && my <= 32 && lay.st >= 8 &&
           (tiles * lay.st + 8) * 8 < (int64_t)kBufferSkip;
}

#define FNO_ROWREG_DISPATCH(FN, ...)                                                                   \
    if (log2H == 7 && log2W == 7) return my <= 16 ? FN<7, 7, 16>(__VA_ARGS__) : FN<7, 7, 32>(__VA_ARGS__); \
    if (log2H == 6 && log2W == 6) return my <= 16 ? FN<6, 6, 16>(__VA_ARGS__) : FN<6, 6, 32>(__VA_ARGS__); \
    if (log2H == 7 && log2W == 6) return my <= 16 ? FN<7, 6, 16>(__VA_ARGS__) : FN<7, 6, 32>(__VA_ARGS__); \
    if (log2H == 6 && log2W == 7) return my <= 16 ? FN<6, 7, 16>(__VA_ARGS__) : FN<6, 7, 32>(__VA_ARGS__); \
    return hipErrorInvalidValue;

hipError_t launch_fwd2d_rowreg(const float* x, float2* xh, const SpecLayout& lay, int64_t nimg, int log2H,
                               int log2W, int mx, int my, const float2* tw, hipStream_t s, const float2* mask) {
    if (!rowreg2d_supported(log2H, log2W, mx, my, lay) || nimg >= INT32_MAX) return hipErrorInvalidValue;
    // the mask's byte range (2 mx my C complex) stays below the buffer range limit
    if (mask && (int64_t)2 * mx * my * lay.C * 8 >= (int64_t)kBufferSkip) return hipErrorInvalidValue;
    const ImageBase ib = image_base(lay);
    const int st = (int)lay.st;
    FNO_ROWREG_DISPATCH(launch_fwd_one, x, xh, ib, st, nimg, mx, my, tw, s, mask)
}

hipError_t launch_inv2d_rowreg(const float2* yh, float* out, const SpecLayout& lay, int64_t nimg, int log2H,
                               int log2W, int mx, int my, const float2* tw, hipStream_t s, const Epilogue& epi) {
    if (!rowreg2d_supported(log2H, log2W, mx, my, lay) || nimg >= INT32_MAX) return hipErrorInvalidValue;
    const ImageBase ib = image_base(lay);
    const int st = (int)lay.st;
    FNO_ROWREG_DISPATCH(launch_inv_one, yh, out, ib, st, nimg, mx, my, tw, s, epi)
}
#undef FNO_ROWREG_DISPATCH

}  // namespace fno
