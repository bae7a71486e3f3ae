// Per-image 2D transforms for grids of 128 x 256 and of 256 or 512 rows by
// 128, 256 or 512 columns with at most 32 (16 at 512 rows) kept columns: the
// row pass and the column pass of one image in one workgroup, the row
// spectrum kept in LDS between them
// (TurboFNO blog, section 2.1: the truncated spectrum stays on chip between
// the passes of the 2D transform; section 2.2: only the kept modes are ever
// formed).
//
// Forward: a workgroup of 16 waves takes one image.  Row pass: each wave
// transforms 64 / LW rows at a time as the short-row kernels do (lane n1 < LW
// of a row holds its samples n1 + LW n2, n2 < 16, and runs a 16-point real
// DFT; the kept bins are formed by binary trees over the phases) and writes
// the bins ky < my of its rows into an LDS plane [H][33] ([H][17] at 512
// rows).  Column pass: the
// kept columns in blocks of 16, thread (n1, c) of 16 LH per block holding
// column c's samples n1 + LH n2 (n2 < 16) of the plane, a 16-point DFT, the
// residues staged in LDS, and every kept mode kx formed by a binary tree
// over the phases, stored to the canonical spectrum [image][2 mx][my].
// Inverse: the same two passes backwards: the kept modes of each column
// block (zero-filled) give the columns of the plane by the residue sums of
// the short-column inverse, and the short-row inverse turns each plane row
// into the image row, with the fused layer epilogue when asked.
// 2 mx must be a multiple of 16 (kept mode q has residue q mod 16) and at
// most 128 (64 at 128 rows); the grid is persistent, one image per workgroup at a time.
#include "fno_device.hpp"
#include "fno_internal.hpp"
#include "fno_realbins.hpp"

namespace fno {
namespace {

constexpr int kS2Threads = 1024;
constexpr int kS2Waves = kS2Threads / 64;
constexpr int kS2MaxKept = 128;      // 2 mx

// kept kx at most: 128, or half the rows at 128 rows (the column twiddles of
// two reading roles per thread then fit the registers)
constexpr int s2_kept(int H) { return H >= 256 ? kS2MaxKept : H / 2; }

template <int LW, int LH>
struct S2Plan {
    static constexpr int W = 16 * LW, H = 16 * LH, Q = 16, NZ = 8, SROWS = NZ + 1;
    // row pass (the short-row forward's roles)
    static constexpr int RPW = 64 / LW;                 // rows per wave
    static constexpr int PBS = LW < 16 ? LW : 16;       // phases per block
    static constexpr int PB = LW / PBS;                 // blocks per row
    static constexpr int SS = LW + PB;                  // row stage stride
    static constexpr int NSL = RPW * PB;                // slots
    static constexpr int BPS = 64 / NSL;                // bins per slot
    static constexpr int RSTAGE = RPW * SROWS * SS;     // row stage per wave
    static constexpr int RPI = kS2Waves * RPW;          // rows per iteration of the workgroup
    // column pass (the short-column forward's roles)
    static constexpr int C = 16;
    static constexpr int PBSc = LH < 16 ? LH : 16;
    static constexpr int PBc = LH / PBSc;
    static constexpr int SSc = LH + PBc;
    static constexpr int NTc = 16 * LH;                 // threads per column block
    static constexpr int NRDc = 16 * C * PBc / NTc;     // reading roles per thread
    static constexpr int CSTAGE = 16 * C * SSc;         // column stage per block
    static constexpr int MPR = s2_kept(H) / 16;         // kept modes per residue, at most
    static constexpr int KS = s2_kept(H) + 2;           // inverse table row stride (16-byte multiple)
    // kept columns: two blocks of 16 (my <= 32), one at 512 rows (my <= 16,
    // so that the plane fits the LDS beside the stages)
    static constexpr int CB = H >= 512 ? 1 : 2;
    static constexpr int PS = 16 * CB + 1;              // plane row stride (complex): odd, rows on distinct bank pairs
    static constexpr int STAGE = kS2Waves * RSTAGE > CB * CSTAGE ? kS2Waves * RSTAGE : CB * CSTAGE;
    static_assert(H % RPI == 0, "whole row iterations");
    static_assert(CB * NTc <= kS2Threads, "column blocks");
};

// ---- forward ------------------------------------------------------------------
template <int LW, int LH>
__global__ __launch_bounds__(kS2Threads) void k_fwd2d_short(const float* __restrict__ x, float2* __restrict__ xh,
                                                            int64_t nimg, int mx, int my, float scale,
                                                            const float2* __restrict__ tw) {
    using P = S2Plan<LW, LH>;
    constexpr int W = P::W, H = P::H, Q = P::Q, NZ = P::NZ, SROWS = P::SROWS;
    constexpr int RPW = P::RPW, PBS = P::PBS, PB = P::PB, SS = P::SS, NSL = P::NSL, BPS = P::BPS;
    constexpr int C = P::C, PBSc = P::PBSc, PBc = P::PBc, SSc = P::SSc, NTc = P::NTc, NRDc = P::NRDc;
    constexpr int MPR = P::MPR, CB = P::CB, PS = P::PS;
    __shared__ float2 plane[H * PS];
    __shared__ float2 stage[P::STAGE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nk = 2 * mx;
    const int nm = nk / 16;

    // row roles: loading lane (row rw of the wave's rows, phase n1); reading
    // lane (phase block pb, item group g; slot s holds item s 64/PB + g =
    // (row it mod RPW, bin it div RPW))
    const int rw = lane / LW, n1 = lane % LW;
    const int pb = lane % PB, g = lane / PB;
    auto item = [&](int sl, int& rr, int& k) __attribute__((always_inline)) {
        const int it = sl * (64 / PB) + g;
        rr = it % RPW;
        k = it / RPW;
    };
    // W^k of each slot's bin; with 128-point rows (eight slots, which would
    // not fit the registers beside the column factors) only the lane's part
    // W^{g / RPW} is kept and the slot's part W^{PBS sl}, the same in every
    // lane, is read where it is used (bin k = PBS sl + g / RPW)
    constexpr bool WKL = LW == 8;
    constexpr int NWK = WKL ? 1 : NSL;
    float2 wk[NWK], vk[PB == 2 ? NSL : 1];
    if constexpr (WKL) wk[0] = tw[((g / RPW) * (kNMax / W)) & (kNMax - 1)];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
        int rr, k;
        item(sl, rr, k);
        const bool cj = k % Q > NZ;
        const float2 w = tw[(k * (kNMax / W)) & (kNMax - 1)];
        if constexpr (!WKL) wk[sl] = cj ? conj2(w) : w;
        if constexpr (PB == 2) {
            const float2 u = cscale(tw[(PBS * pb * k * (kNMax / W)) & (kNMax - 1)], 0.5f);
            vk[sl] = cj ? conj2(u) : u;
        }
    }
    float2* const rstage = stage + wave * P::RSTAGE;

    // column roles: block cb, thread tl of the block: loading (column c,
    // phase m1); reading role rho = tl + NTc h (block pbc, column cr, residue
    // rr)
    const int cb = tid / NTc, tl = tid % NTc;
    const bool col_thread = cb < CB;
    const int c = tl % C, m1 = tl / C;
    auto role = [&](int h, int& pbc, int& cr, int& rr) __attribute__((always_inline)) {
        const int rho = tl + NTc * h;
        pbc = rho % PBc;
        cr = (rho / PBc) % C;
        rr = rho / (PBc * C);
    };
    // W^k of the role's modes (with two phase blocks, the second block's
    // factor W^{16 k} is the tree's last square squared once more)
    float2 wc[NRDc][MPR];
#pragma unroll
    for (int h = 0; h < NRDc; ++h) {
        int pbc, cr, rr;
        role(h, pbc, cr, rr);
#pragma unroll
        for (int i = 0; i < MPR; ++i) {
            const int q = rr + 16 * i;
            const int k = q < nk ? (q < mx ? q : H - nk + q) : 0;
            wc[h][i] = tw[((int64_t)k * (kNMax / H)) & (kNMax - 1)];
        }
    }
    float2* const cstage = stage + (col_thread ? cb : 0) * P::CSTAGE;

    for (int64_t img = blockIdx.x; img < nimg; img += gridDim.x) {
#pragma unroll
        for (int sl = 0; sl < NWK; ++sl) asm volatile("" : "+v"(wk[sl].x), "+v"(wk[sl].y));
        const float* const ximg = x + img * (int64_t)(H * W);
        // ---- row pass: bins ky < my of every row into the plane --------------
        for (int row0 = wave * RPW; row0 < H; row0 += P::RPI) {
            const float* src = ximg + (row0 + rw) * W + n1;
            float2 z[NZ];
#pragma unroll
            for (int m = 0; m < NZ; ++m) z[m] = make_float2(src[LW * (2 * m)], src[LW * (2 * m + 1)]);
            dft<NZ, -1>(z);
            static_for<0, SROWS>([&](auto r) { rstage[(rw * SROWS + r) * SS + n1 + n1 / PBS] = real_bin2<Q, r>(z); });
            wave_lds_sync();
            static_for<0, NSL>([&](auto sl) {
                if (BPS * sl < my) {             // uniform: a slot with a kept bin
                    int rr, k;
                    item(sl, rr, k);
                    const int r = k % Q;
                    const bool cj = r > NZ;
                    const float2* const sp = rstage + (rr * SROWS + (cj ? Q - r : r)) * SS + (PBS + 1) * pb;
                    float2 v[PBS];
#pragma unroll
                    for (int t = 0; t < PBS; ++t) v[t] = sp[t];
                    float2 w;
                    if constexpr (WKL) {
                        w = cmul(wk[0], tw[(PBS * sl * (kNMax / W)) & (kNMax - 1)]);
                        if (cj) w = conj2(w);
                    } else {
                        w = wk[sl];
                    }
#pragma unroll
                    for (int len = PBS; len > 1; len /= 2) {
#pragma unroll
                        for (int t = 0; t < len / 2; ++t) v[t] = cfma(v[2 * t], w, v[2 * t + 1]);
                        if (len > 2) w = cmul(w, w);
                    }
                    float2 acc;
                    if constexpr (PB == 2) {
                        acc = cmul(vk[sl], v[0]);
                        acc.x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.x), 0xB1, 0xF, 0xF, false));
                        acc.y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.y), 0xB1, 0xF, 0xF, false));
                    } else {
                        acc = cscale(v[0], 0.5f);
                    }
                    if (pb == 0 && k < my) plane[(row0 + rr) * PS + k] = cj ? conj2(acc) : acc;
                }
            });
            wave_lds_sync();                    // the stage is read before the next rows overwrite it
        }
        __syncthreads();                        // every row is in the plane (and the row stages are free)

        // ---- column pass: the kept modes of the kept columns -----------------
        if (col_thread && C * cb < my) {
            const int kyc = C * cb + c < my ? C * cb + c : my - 1;
            float2 v[16];
#pragma unroll
            for (int n2 = 0; n2 < 16; ++n2) v[n2] = plane[(m1 + LH * n2) * PS + kyc];
            dft<16, -1>(v);
#pragma unroll
            for (int q = 0; q < 16; ++q) cstage[(q * C + c) * SSc + m1 + m1 / PBSc] = v[q];
        }
        __syncthreads();
        if (col_thread && C * cb < my) {
            float2* const dst = xh + img * (int64_t)nk * my + C * cb;
#pragma unroll
            for (int h = 0; h < NRDc; ++h) {
                int pbc, cr, rr;
                role(h, pbc, cr, rr);
                const float2* const sp = cstage + (rr * C + cr) * SSc + (PBSc + 1) * pbc;
                float2 sv[PBSc];
#pragma unroll
                for (int t = 0; t < PBSc; ++t) sv[t] = sp[t];
                const bool store = pbc == 0 && C * cb + cr < my;
#pragma unroll
                for (int i = 0; i < MPR; ++i) {
                    if (i < nm) {                // uniform
                        float2 u[PBSc / 2];
                        float2 w = wc[h][i];
#pragma unroll
                        for (int t = 0; t < PBSc / 2; ++t) u[t] = cfma(sv[2 * t], w, sv[2 * t + 1]);
#pragma unroll
                        for (int len = PBSc / 2; len > 1; len /= 2) {
                            w = cmul(w, w);
#pragma unroll
                            for (int t = 0; t < len / 2; ++t) u[t] = cfma(u[2 * t], w, u[2 * t + 1]);
                        }
                        float2 acc;
                        if constexpr (PBc == 2) {
                            // w is W^{8k} here
                            const float2 f = pbc ? cscale(cmul(w, w), scale) : make_float2(scale, 0.0f);
                            acc = cmul(f, u[0]);
                            acc.x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.x), 0xB1, 0xF, 0xF, false));
                            acc.y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.y), 0xB1, 0xF, 0xF, false));
                        } else {
                            acc = cscale(u[0], scale);
                        }
                        if (store) dst[(int64_t)(rr + 16 * i) * my + cr] = acc;
                        // one mode at a time (the next mode's tree starts
                        // from a factor defined after this mode's result)
                        if (i + 1 < MPR)
                            asm volatile("" : "+v"(wc[h][i + 1].x), "+v"(wc[h][i + 1].y) : "v"(acc.x), "v"(acc.y));
                    }
                }
            }
        }
        __syncthreads();                        // the plane and the stage are free for the next image
    }
}

// ---- inverse ------------------------------------------------------------------
// NJ: the 16-bin groups of a row that can hold a kept bin (my <= 16 NJ).
template <int LW, int LH, bool EPI, int NJ>
__global__ __launch_bounds__(kS2Threads) void k_inv2d_short(const float2* __restrict__ yh, float* __restrict__ out,
                                                            int64_t nimg, int mx, int my, float scale,
                                                            const float2* __restrict__ tw, Epilogue epi) {
    using P = S2Plan<LW, LH>;
    constexpr int W = P::W, H = P::H, Q = P::Q, NZ = P::NZ;
    constexpr int RPW = P::RPW, C = P::C, NTc = P::NTc, KS = P::KS;
    constexpr int CB = P::CB, PS = P::PS;
    constexpr int TF = NZ + 5;                 // residue-factor table row (odd: phases on distinct bank pairs)
    static_assert(NJ <= CB, "at most 16 CB kept columns");
    __shared__ float2 plane[H * PS];
    __shared__ __align__(16) float2 T[LH * KS];           // [m1][q]: W_H^{-m1 k_q}
    __shared__ __align__(16) float2 xs[CB * C * KS];   // [block][c][q]: the image's kept modes
    __shared__ float2 ftab[LW * TF];                      // [n1][t]: row residue factors
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nk = 2 * mx;

    // per-workgroup tables: the kept modes' column twiddles, and the row
    // residue factors W_W^{n1 r} scale (r <= Q/2; X[0] is halved in the
    // plane, so every bin counts twice and 2 (scale / 2) = scale) and
    // W_LW^{n1 j} (entries Q/2 + j)
    for (int e = tid; e < LH * nk; e += kS2Threads) {
        const int m = e / nk, q = e % nk;
        const int k = q < mx ? q : H - nk + q;
        T[m * KS + q] = conj2(tw[((int64_t)m * k * (kNMax / H)) & (kNMax - 1)]);
    }
    for (int e = tid; e < LW * TF; e += kS2Threads) {
        const int nn = e / TF, t = e % TF;
        ftab[e] = t <= NZ ? cscale(tw[(nn * t * (kNMax / W)) & (kNMax - 1)], scale)
                          : tw[(16 * nn * (t - NZ) * (kNMax / W)) & (kNMax - 1)];
    }
    __syncthreads();

    // column roles: block cb, phase m1, column c
    const int cb = tid / NTc, tl = tid % NTc;
    const bool col_thread = cb < CB;
    const int c = tl % C, m1 = tl / C;
    const float2* const tp = T + m1 * KS;
    const float2* const xp = xs + ((col_thread ? cb : 0) * C + c) * KS;
    // row roles: row rw of the wave's rows, phase n1
    const int rw = lane / LW, n1 = lane % LW;
    const float2* const ft = ftab + n1 * TF;
    auto res = [&](auto r) __attribute__((always_inline)) {
        if constexpr (r <= NZ) return ft[r];
        else return cmul(ft[NZ + 1], conj2(ft[r <= NZ ? 0 : Q - r]));
    };

    for (int64_t img = blockIdx.x; img < nimg; img += gridDim.x) {
        // ---- the image's kept modes (zero past my), column fastest --------
        const float2* const src = yh + img * (int64_t)nk * my;
        for (int e = tid; e < nk * CB * C; e += kS2Threads) {
            const int q = e / (CB * C), col = e % (CB * C);
            xs[col * KS + q] = col < my ? src[(int64_t)q * my + col] : make_float2(0.0f, 0.0f);
        }
        __syncthreads();
        // ---- column pass: the plane's columns ky < 16 NJ ------------------
        if (col_thread && C * cb < my) {
            float2 v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = make_float2(0.0f, 0.0f);
            static_for<0, s2_kept(H) / 16>([&](auto ch) {
                if (16 * ch < nk) {              // uniform
                    static_for<0, 8>([&](auto pp) {
                        constexpr int q = 16 * ch + 2 * pp;
                        const float4 t2 = *reinterpret_cast<const float4*>(tp + q);
                        const float4 x2 = *reinterpret_cast<const float4*>(xp + q);
                        v[2 * pp] = cfma(v[2 * pp], make_float2(t2.x, t2.y), make_float2(x2.x, x2.y));
                        v[2 * pp + 1] = cfma(v[2 * pp + 1], make_float2(t2.z, t2.w), make_float2(x2.z, x2.w));
                    });
                }
            });
            dft<16, 1>(v);
            const int ky = C * cb + c;
#pragma unroll
            for (int n2 = 0; n2 < 16; ++n2) {
                // the row transform's input: zero past my, the DC bin halved
                // with its imaginary part dropped
                float2 o = ky < my ? v[n2] : make_float2(0.0f, 0.0f);
                if (ky == 0) o = make_float2(0.5f * o.x, 0.0f);
                plane[(m1 + LH * n2) * PS + ky] = o;
            }
        }
        __syncthreads();                        // the plane is whole (and the modes are read)
        // ---- row pass: each plane row to its image row ----------------------
        for (int row0 = wave * RPW; row0 < H; row0 += P::RPI) {
            const float2* const xr = plane + (row0 + rw) * PS;
            float2 V[Q], cur[NJ], nxt[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j) cur[j] = xr[Q * j];
            static_for<0, Q>([&](auto r) {
                if constexpr (r + 1 < Q) {
#pragma unroll
                    for (int j = 0; j < NJ; ++j) nxt[j] = xr[r + 1 + Q * j];
                }
                float2 acc = cur[0];
                static_for<1, NJ>([&](auto j) { acc = cfma(acc, cur[j], conj2(ft[NZ + j])); });
                V[r] = cmul(acc, conj2(res(r)));
                asm volatile("" : "+v"(V[r].x), "+v"(V[r].y) : : "memory");
#pragma unroll
                for (int j = 0; j < NJ; ++j) cur[j] = nxt[j];
            });
            float2 Hh[NZ + 1];
#pragma unroll
            for (int r = 0; r <= NZ; ++r) {
                const float2 a = V[r], b = V[(Q - r) % Q];
                Hh[r] = make_float2(a.x + b.x, a.y - b.y);
            }
            float2 z[NZ];
            static_for<0, NZ>([&](auto k) { z[k] = packed_bin<Q, k>(Hh); });
            dft<NZ, 1>(z);
            const int64_t grow0 = img * H + row0;   // the wave's first row in the whole output
            float* const dst = out + (grow0 + rw) * W + n1;
            if constexpr (EPI) {
                const uint32_t urow0 = __builtin_amdgcn_readfirstlane((uint32_t)grow0);
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(epi.branch ? epi.branch + (int64_t)urow0 * W : out,
                                                            epi.branch ? (uint32_t)(RPW * W * 4) : 0u);
                const float bias = epi_bias(epi, urow0 + rw);
                float br[2 * NZ];
#pragma unroll
                for (int k = 0; k < 2 * NZ; ++k) br[k] = buffer_load_f1(rb, (uint32_t)(rw * W + n1 + LW * k) * 4u, 0);
#pragma unroll
                for (int m = 0; m < NZ; ++m) {
                    nt_store(&dst[LW * (2 * m)], epi_apply(epi, z[m].x, bias, br[2 * m]));
                    nt_store(&dst[LW * (2 * m + 1)], epi_apply(epi, z[m].y, bias, br[2 * m + 1]));
                }
            } else {
#pragma unroll
                for (int m = 0; m < NZ; ++m) {
                    nt_store(&dst[LW * (2 * m)], z[m].x);
                    nt_store(&dst[LW * (2 * m + 1)], z[m].y);
                }
            }
        }
        __syncthreads();                        // the plane and the modes are free for the next image
    }
}

template <typename K>
hipError_t launch_s2(K kernel, int64_t nimg, hipStream_t s, int& g) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kS2Threads, 0);
    if (e != hipSuccess) return e;
    int64_t n = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    if (n > nimg) n = nimg;
    g = (int)n;
    (void)s;
    return hipSuccess;
}

}  // namespace

// 128 rows of 256 points, 256 or 512 rows of 128, 256 or 512 points (the
// forms that fit the registers of 16 waves without spills); at 512 rows at
// most 16 kept columns (the plane beside the stages in the LDS)
bool short2d_supported(int log2H, int log2W, int mx, int my) {
    return log2H >= 7 && log2H <= 9 && (log2W == 8 || (log2W == 9 && log2H > 7) || (log2W == 7 && log2H > 7)) &&
           my >= 1 &&
           my <= (log2H == 9 ? 16 : 32) &&
           mx >= 1 && (2 * mx) % 16 == 0 && 2 * mx <= s2_kept(1 << log2H);
}

// One image per workgroup and one workgroup per CU: with fewer images than
// half the CUs the staged kernels, which spread an image over several
// workgroups, were faster (256 x 256, 32 and 64 images: 37 against 28 and
// 32 us; even at 128 images, faster from 256 on).  With 128-point rows the
// one-kernel form pays only up to one image per CU at 256 rows (128 and 256
// images 25 and 31 us against 30 and 35 staged; 512 images 50 against 50
// with 16 kept columns, 46.5 against 43 with 8) and up to one image per two
// CUs at 512 rows (128 images 34 against 39 us; 192 and 256 images the same
// as staged).
bool short2d_pays(int64_t nimg, int log2H, int log2W) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    return 2 * nimg >= cus && (log2W != 7 || nimg <= (log2H == 9 ? cus / 2 : cus));
}

hipError_t launch_fwd2d_short(const float* x, float2* xh, int64_t nimg, int log2H, int log2W, int mx, int my,
                              float scale, const float2* tw, hipStream_t s) {
    if (!short2d_supported(log2H, log2W, mx, my) || nimg <= 0 || nimg >= INT32_MAX) return hipErrorInvalidValue;
    auto go = [&](auto kernel) {
        int g = 0;
        const hipError_t e = launch_s2(kernel, nimg, s, g);
        if (e != hipSuccess) return e;
        return launch_kernel(kernel, dim3((unsigned)g), dim3(kS2Threads), 0, s, x, xh, nimg, mx, my, scale, tw);
    };
    if (log2H == 9) {
        if (log2W == 7) return go(k_fwd2d_short<8, 32>);
        return log2W == 8 ? go(k_fwd2d_short<16, 32>) : go(k_fwd2d_short<32, 32>);
    }
    if (log2H == 7) return go(k_fwd2d_short<16, 8>);
    if (log2W == 7) return go(k_fwd2d_short<8, 16>);
    if (log2W == 8) return go(k_fwd2d_short<16, 16>);
    return go(k_fwd2d_short<32, 16>);
}

hipError_t launch_inv2d_short(const float2* yh, float* out, int64_t nimg, int log2H, int log2W, int mx, int my,
                              float scale, const float2* tw, hipStream_t s, const Epilogue& epi) {
    if (!short2d_supported(log2H, log2W, mx, my) || nimg <= 0 || nimg >= INT32_MAX) return hipErrorInvalidValue;
    auto go = [&](auto kernel) {
        int g = 0;
        const hipError_t e = launch_s2(kernel, nimg, s, g);
        if (e != hipSuccess) return e;
        return launch_kernel(kernel, dim3((unsigned)g), dim3(kS2Threads), 0, s, yh, out, nimg, mx, my, scale, tw,
                             epi);
    };
    const bool two = my > 16;
    if (log2H == 7) {                       // W = 256
        if (epi.on) return two ? go(k_inv2d_short<16, 8, true, 2>) : go(k_inv2d_short<16, 8, true, 1>);
        return two ? go(k_inv2d_short<16, 8, false, 2>) : go(k_inv2d_short<16, 8, false, 1>);
    }
    if (log2H == 9) {                       // my <= 16
        if (log2W == 7) return epi.on ? go(k_inv2d_short<8, 32, true, 1>) : go(k_inv2d_short<8, 32, false, 1>);
        if (log2W == 8) return epi.on ? go(k_inv2d_short<16, 32, true, 1>) : go(k_inv2d_short<16, 32, false, 1>);
        return epi.on ? go(k_inv2d_short<32, 32, true, 1>) : go(k_inv2d_short<32, 32, false, 1>);
    }
    if (log2W == 7) {                       // H = 256
        if (epi.on) return two ? go(k_inv2d_short<8, 16, true, 2>) : go(k_inv2d_short<8, 16, true, 1>);
        return two ? go(k_inv2d_short<8, 16, false, 2>) : go(k_inv2d_short<8, 16, false, 1>);
    }
    if (log2W == 8) {
        if (epi.on) return two ? go(k_inv2d_short<16, 16, true, 2>) : go(k_inv2d_short<16, 16, true, 1>);
        return two ? go(k_inv2d_short<16, 16, false, 2>) : go(k_inv2d_short<16, 16, false, 1>);
    }
    if (epi.on) return two ? go(k_inv2d_short<32, 16, true, 2>) : go(k_inv2d_short<32, 16, true, 1>);
    return two ? go(k_inv2d_short<32, 16, false, 2>) : go(k_inv2d_short<32, 16, false, 1>);
}

}  // namespace fno
