// Pruned column transforms for tall grids (H = 64 Q rows, Q in {4, 8, 16, 32};
// 256 and 512 rows with 2 mx a multiple of 16 take the short-column kernels
// further down)
// when at most 64 kx are kept on each side and my <= 64 columns exist:
// the forward one computes only kx in [0,mx) u [H-mx,H), the inverse one
// starts from those alone (TurboFNO blog, sections 2.1-2.2: the second 1D
// transform of the 2D one, restricted to the kept modes).
//
// Row h of an image's row spectrum R[H][my] is split h = n1 + 64 n2
// (n1 < 64, n2 < Q).  With W = exp(-2 pi i / H):
//   X[k] = sum_n1 W^{n1 k} Y_n1[k mod Q],   Y_n1 = DFT_Q over n2 of R[n1 + 64 n2],
//   R'[n1 + 64 n2] = sum_r W_Q^{-n2 r} V_n1[r],   V_n1[r] = sum_{kept k = r mod Q} W^{-n1 k} X[k].
// A workgroup of 512 threads takes one image and 8 neighbouring columns;
// thread (n1, c) holds column c's samples n1 + 64 n2 (so a wave's loads and
// stores touch eight 64-byte runs) and runs its Q-point DFT in registers.
// 2 mx must be a multiple of Q: then a kept mode's residue mod Q is its
// index's, and every register index is static.
// Forward: every Y_n1[r] is staged in LDS once; a reading lane (residue r,
// column, quarter p of the phases) sums its 16 phases n1 = 16 p + t for four
// kept modes k of that residue at once, as
//   W^{16 p k} sum_t (W^k)^t Y_{16 p + t}[r]
// (a binary tree with the factors W^k, W^2k, W^4k, W^8k), and the quarters
// are added across the lane quad.
// Inverse: the twiddles W^{-n1 k} of the kept modes are tabulated once per
// workgroup in LDS from the host-built table; each thread accumulates its
// V_n1[r] from the kept modes in LDS.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kColThreads = 512;
constexpr int kColC = 8;                 // columns per workgroup
constexpr int kMaxKept = 128;            // 2 mx

// Twiddle table T[q][n1] = W^{n1 k_q} for the kept modes k_q (q < 2 mx),
// and up to the end of the last 8-mode chunk (the accumulation below runs
// whole chunks; those entries meet zeroed modes).  Every thread issues all
// of its (at most 16) table reads before it writes any entry, so the
// gathers overlap instead of queueing one by one.
template <int H>
__device__ __forceinline__ void fill_twiddles(float2* T, int mx, const float2* __restrict__ tw, int sign) {
    constexpr int kPer = kMaxKept * 64 / kColThreads;
    const int ne = (2 * mx + 7) / 8 * 8 * 64;
    float2 w[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = threadIdx.x + kColThreads * j;
        const int q = e >> 6, n1 = e & 63;
        const int k = q < mx ? q : H - 2 * mx + q;
        if (e < ne) w[j] = tw[((int64_t)n1 * k * (kNMax / H)) & (kNMax - 1)];
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = threadIdx.x + kColThreads * j;
        if (e < ne) T[e] = make_float2(w[j].x, sign > 0 ? -w[j].y : w[j].y);
    }
}

constexpr int kColStage = 68;            // forward stage row stride (complex): 64 phases + pad

// index of (stage row, phase n1) in the forward stage
__device__ __forceinline__ int col_stage_at(int row, int n1) { return row * kColStage + n1 + (n1 >> 4); }

template <int Q>
__global__ __launch_bounds__(kColThreads) void k_cols_fwd_pruned(const float2* __restrict__ r,
                                                                 float2* __restrict__ xh, int nkb, int mx, int my,
                                                                 float scale, const float2* __restrict__ tw) {
    constexpr int H = 64 * Q;
    constexpr int NRH = 2;                           // reading roles per thread
    __shared__ float2 stage[Q * kColC * kColStage];  // row (residue r, column c): Y_n1[r] of the 64 phases
    const int tid = threadIdx.x;
    const int c = tid & 7;                           // column within the block
    const int n1 = tid >> 3;                         // row phase
    // column blocks 2j and 2j + 1 (the two halves of every 128-byte line of
    // the row spectrum) go to workgroups on the same XCD at the same time,
    // so that L2 fetches each line once
    const int64_t blk = paired_image(blockIdx.x, (int64_t)gridDim.x);
    const int64_t img = blk / nkb;
    const int ky0 = (int)(blk % nkb) * kColC;
    const int ky = ky0 + c;
    const int kyc = ky < my ? ky : my - 1;
    const int nk = 2 * mx;

    // column samples n1 + 64 n2 (issued first, so that the twiddles below
    // are fetched while they are in flight)
    const float2* src = r + img * (int64_t)H * my + kyc;
    float2 v[Q];
#pragma unroll
    for (int n2 = 0; n2 < Q; ++n2) v[n2] = src[(int64_t)(n1 + 64 * n2) * my];

    // Reading role rho = tid + 512 h: quad lane p = rho & 3, column
    // cr = (rho >> 2) & 7, residue group g = rho >> 5 (residue g mod Q, kept
    // modes q = g mod Q + Q (4 (g div Q) + b), b < 4; 2 mx <= 128 gives at
    // most 32 groups).  Kept mode q is k_q = q or H - 2 mx + q; modes past
    // 2 mx take k = 0 and are not stored.
    float2 wk[NRH][4], vk[NRH][4];
#pragma unroll
    for (int h = 0; h < NRH; ++h) {
        const int rho = tid + kColThreads * h;
        const int p = rho & 3, g = rho >> 5;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int q = g % Q + Q * (4 * (g / Q) + b);
            const int k = q < nk ? (q < mx ? q : H - nk + q) : 0;
            wk[h][b] = tw[((int64_t)k * (kNMax / H)) & (kNMax - 1)];
            vk[h][b] = cscale(tw[((int64_t)16 * p * k * (kNMax / H)) & (kNMax - 1)], scale);
        }
    }
    dft<Q, -1>(v);
#pragma unroll
    for (int rr = 0; rr < Q; ++rr) stage[col_stage_at(rr * kColC + c, n1)] = v[rr];
    __syncthreads();

    float2* const dst = xh + img * (int64_t)nk * my;
#pragma unroll
    for (int h = 0; h < NRH; ++h) {
        const int rho = tid + kColThreads * h;
        const int p = rho & 3, cr = (rho >> 2) & 7, g = rho >> 5;
        const int rr = g % Q;
        const float2* const srow = stage + col_stage_at(rr * kColC + cr, 16 * p);
        float2 s16[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) s16[t] = srow[t];
        // first level of every mode's tree (s16 is dead after it), then the
        // rest of each tree
        float2 u[4][8];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int t = 0; t < 8; ++t) u[b][t] = cfma(s16[2 * t], wk[h][b], s16[2 * t + 1]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float2 w2 = cmul(wk[h][b], wk[h][b]);
            const float2 w4 = cmul(w2, w2);
            const float2 w8 = cmul(w4, w4);
#pragma unroll
            for (int t = 0; t < 4; ++t) u[b][t] = cfma(u[b][2 * t], w2, u[b][2 * t + 1]);
#pragma unroll
            for (int t = 0; t < 2; ++t) u[b][t] = cfma(u[b][2 * t], w4, u[b][2 * t + 1]);
            const float2 acc = quad_sum(cmul(vk[h][b], cfma(u[b][0], w8, u[b][1])));
            const int q = rr + Q * (4 * (g / Q) + b);
            if (p == 0 && q < nk && ky0 + cr < my) dst[(int64_t)q * my + ky0 + cr] = acc;
        }
    }
}

template <int Q>
__global__ __launch_bounds__(kColThreads) void k_cols_inv_pruned(const float2* __restrict__ yh,
                                                                 float2* __restrict__ r, int nkb, int mx, int my,
                                                                 const float2* __restrict__ tw) {
    constexpr int H = 64 * Q;
    __shared__ float2 T[kMaxKept * 64];              // 64 KiB: conj twiddles
    __shared__ float2 xs[kMaxKept * kColC];          // the block's kept modes, [q][c]
    const int tid = threadIdx.x;
    const int c = tid & 7;
    const int n1 = tid >> 3;
    // column blocks 2j and 2j + 1 (the two halves of every 128-byte line of
    // the row spectrum) go to workgroups on the same XCD at the same time,
    // so that L2 writes each line back whole
    const int64_t blk = paired_image(blockIdx.x, (int64_t)gridDim.x);
    const int64_t img = blk / nkb;
    const int ky0 = (int)(blk % nkb) * kColC;
    const int ky = ky0 + c;
    const int nk = 2 * mx;

    fill_twiddles<H>(T, mx, tw, 1);
    const float2* src = yh + img * (int64_t)nk * my;
    // the kept modes, zero up to the end of the last 8-mode chunk (2 mx is a
    // multiple of Q, which is 4 at H = 256: not always of 8)
    const int nk8 = (nk + 7) / 8 * 8;
    for (int e = tid; e < nk8 * kColC; e += kColThreads) {
        const int q = e >> 3, cc = e & 7;
        xs[e] = q < nk && ky0 + cc < my ? src[(int64_t)q * my + ky0 + cc] : make_float2(0.0f, 0.0f);
    }
    __syncthreads();
    // V[r] = sum_{kept k = r mod Q} W^{-n1 k} X[k]; k_q mod Q = q mod Q
    // because 2 mx is a multiple of Q
    float2 v[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j) v[j] = make_float2(0.0f, 0.0f);
    static_for<0, kMaxKept / 8>([&](auto ch) {
        if (8 * ch < nk) {
            static_for<0, 8>([&](auto kk) {
                constexpr int q = 8 * ch + kk;
                const float2 u = cmul(T[q * 64 + n1], xs[q * kColC + c]);
                v[q % Q] = cadd(v[q % Q], u);
            });
        }
    });
    dft<Q, 1>(v);
    if (ky < my) {
        float2* dst = r + img * (int64_t)H * my + ky;
#pragma unroll
        for (int n2 = 0; n2 < Q; ++n2) dst[(int64_t)(n1 + 64 * n2) * my] = v[n2];
    }
}

// ---- short columns: H = 16 L rows, L in {4, 8, 16, 32} ---------------------
// At 256 and 512 rows the kernels above hold four or eight samples per
// thread and gather their twiddles per workgroup for 16 KiB of data.  Here
// thread (n1, c) of 16 L holds column c's samples n1 + L n2 (n2 < 16) of a
// block of 16 columns (each load and store instruction covers whole
// 128-byte runs of the row spectrum) and runs a 16-point DFT; the grid is
// persistent, so the twiddles are formed once per thread (forward) or per
// workgroup (inverse) for all the column blocks it walks.  2 mx must be a
// multiple of 16: kept mode q then has the residue q mod 16.
// Forward: every Y_n1[r] is staged in LDS; reading role (residue r, column,
// block of up to 16 phases) forms every kept mode q = r + 16 i of its
// residue as W^{PBS pb k} sum_t (W^k)^t Y_{PBS pb + t}[r] by the binary
// tree above, the two blocks of a 512-row column added across neighbouring
// lanes; with fewer threads than roles (64 and 128 rows) each thread takes
// several.
// Inverse: thread (n1, c) accumulates V_n1[r] = sum_{q = r mod 16}
// W^{-n1 k_q} X[k_q] from a per-workgroup LDS table of the kept modes'
// twiddles and the block's kept modes, then runs its 16-point inverse DFT.
constexpr int kShortC = 16;              // columns per work item

// kept modes at most, for H rows, and the LDS row stride of the inverse
// tables (complex, a 16-byte multiple, rows on distinct bank pairs)
constexpr int short_kept(int H) { return H < kMaxKept ? H : kMaxKept; }
constexpr int short_ks(int H) { return short_kept(H) + 2; }

template <int L>
__global__ __launch_bounds__(16 * L) __attribute__((amdgpu_waves_per_eu(4))) void k_cols_fwd_short(const float2* __restrict__ r, float2* __restrict__ xh,
                                                          int64_t nitems, int nkb, int mx, int my, float scale,
                                                          const float2* __restrict__ tw) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32, "short columns: 64 to 512 rows");
    constexpr int H = 16 * L, C = kShortC, NT = 16 * L;
    constexpr int PBS = L < 16 ? L : 16;             // phases per block
    constexpr int PB = L / PBS;                      // blocks per column
    constexpr int SS = L + PB;                       // stage row stride: a pad after every block
    constexpr int NRD = 16 * C * PB / NT;            // reading roles per thread
    constexpr int MPR = short_kept(H) / 16;          // kept modes per residue, at most
    __shared__ float2 stage[16 * C * SS];            // row (residue, column): the L phases
    const int tid = threadIdx.x;
    const int c = tid % C, n1 = tid / C;             // loading role
    const int nk = 2 * mx;
    const int nm = nk / 16;                          // kept modes per residue
    // reading role rho = tid + NT h: block pb, column cr, residue rr
    auto role = [&](int h, int& pb, int& cr, int& rr) __attribute__((always_inline)) {
        const int rho = tid + NT * h;
        pb = rho % PB;
        cr = (rho / PB) % C;
        rr = rho / (PB * C);
    };
    // W^k of the role's modes, and W^{PBS pb k} (times the output scale)
    // with two blocks per column
    float2 wk[NRD][MPR], vk[PB == 2 ? NRD : 1][MPR];
#pragma unroll
    for (int h = 0; h < NRD; ++h) {
        int pb, cr, rr;
        role(h, pb, cr, rr);
#pragma unroll
        for (int i = 0; i < MPR; ++i) {
            const int q = rr + 16 * i;
            const int k = q < nk ? (q < mx ? q : H - nk + q) : 0;
            wk[h][i] = tw[((int64_t)k * (kNMax / H)) & (kNMax - 1)];
            if constexpr (PB == 2) vk[h][i] = cscale(tw[((int64_t)PBS * pb * k * (kNMax / H)) & (kNMax - 1)], scale);
        }
    }
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
#pragma unroll
        for (int h = 0; h < NRD; ++h)
#pragma unroll
            for (int i = 0; i < MPR; ++i) {
                asm volatile("" : "+v"(wk[h][i].x), "+v"(wk[h][i].y));
                if constexpr (PB == 2) asm volatile("" : "+v"(vk[h][i].x), "+v"(vk[h][i].y));
            }
        const int64_t img = item / nkb;
        const int ky0 = (int)(item % nkb) * C;
        const int kyc = ky0 + c < my ? ky0 + c : my - 1;
        // a uniform image base and 32-bit element offsets (an image holds
        // at most 512 x 64 of them): one address register per load
        const float2* const src = r + img * (int64_t)H * my;
        const uint32_t o0 = (uint32_t)(n1 * my + kyc), os = (uint32_t)(L * my);
        float2 v[16];
#pragma unroll
        for (int n2 = 0; n2 < 16; ++n2) v[n2] = src[o0 + os * (uint32_t)n2];
        dft<16, -1>(v);
#pragma unroll
        for (int q = 0; q < 16; ++q) stage[(q * C + c) * SS + n1 + n1 / PBS] = v[q];
        __syncthreads();
        float2* const dst0 = xh + img * (int64_t)nk * my + ky0;
#pragma unroll
        for (int h = 0; h < NRD; ++h) {
            int pb, cr, rr;
            role(h, pb, cr, rr);
            const float2* const sp = stage + (rr * C + cr) * SS + (PBS + 1) * pb;
            float2 sv[PBS];
#pragma unroll
            for (int t = 0; t < PBS; ++t) sv[t] = sp[t];
            const bool store = pb == 0 && ky0 + cr < my;
#pragma unroll
            for (int i = 0; i < MPR; ++i) {
                if (i < nm) {                            // uniform
                    float2 u[PBS / 2];
                    float2 w = wk[h][i];
#pragma unroll
                    for (int t = 0; t < PBS / 2; ++t) u[t] = cfma(sv[2 * t], w, sv[2 * t + 1]);
#pragma unroll
                    for (int len = PBS / 2; len > 1; len /= 2) {
                        w = cmul(w, w);
#pragma unroll
                        for (int t = 0; t < len / 2; ++t) u[t] = cfma(u[2 * t], w, u[2 * t + 1]);
                    }
                    float2 acc;
                    if constexpr (PB == 2) {
                        acc = cmul(vk[h][i], u[0]);
                        acc.x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.x), 0xB1, 0xF, 0xF, false));
                        acc.y += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc.y), 0xB1, 0xF, 0xF, false));
                    } else {
                        acc = cscale(u[0], scale);
                    }
                    if (store) dst0[(int64_t)(rr + 16 * i) * my + cr] = acc;
                    // one mode at a time: the next mode's tree starts from a
                    // factor defined after this mode's result, so that the
                    // trees do not all run side by side in registers
                    if (i + 1 < MPR)
                        asm volatile("" : "+v"(wk[h][i + 1].x), "+v"(wk[h][i + 1].y) : "v"(acc.x), "v"(acc.y));
                }
            }
        }
        __syncthreads();                                 // the stage is read before the next block overwrites it
    }
}

template <int L>
__global__ __launch_bounds__(16 * L) void k_cols_inv_short(const float2* __restrict__ yh, float2* __restrict__ r,
                                                          int64_t nitems, int nkb, int mx, int my,
                                                          const float2* __restrict__ tw) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32, "short columns: 64 to 512 rows");
    constexpr int H = 16 * L, C = kShortC, NT = 16 * L;
    constexpr int KS = short_ks(H);
    // 16-byte aligned: the mode pairs below are read as one 16-byte word
    __shared__ __align__(16) float2 T[L * KS];   // [n1][q]: W^{-n1 k_q}
    __shared__ __align__(16) float2 xs[C * KS];  // [c][q]: the block's kept modes
    const int tid = threadIdx.x;
    const int c = tid % C, n1 = tid / C;
    const int nk = 2 * mx;
    for (int e = tid; e < L * nk; e += NT) {
        const int n = e / nk, q = e % nk;
        const int k = q < mx ? q : H - nk + q;
        T[n * KS + q] = conj2(tw[((int64_t)n * k * (kNMax / H)) & (kNMax - 1)]);
    }
    const float2* const tp = T + n1 * KS;
    const float2* const xp = xs + c * KS;
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int64_t img = item / nkb;
        const int ky0 = (int)(item % nkb) * C;
        const float2* const src = yh + img * (int64_t)nk * my + ky0;
        // the block's kept modes (column fastest: whole runs of each mode row)
        for (int e = tid; e < nk * C; e += NT) {
            const int q = e / C, cc = e % C;
            xs[cc * KS + q] = ky0 + cc < my ? src[(int64_t)q * my + cc] : make_float2(0.0f, 0.0f);
        }
        __syncthreads();
        float2 v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = make_float2(0.0f, 0.0f);
        // modes in chunks of 16 (q mod 16 static), two per LDS read
        static_for<0, short_kept(H) / 16>([&](auto ch) {
            if (16 * ch < nk) {                          // uniform
                static_for<0, 8>([&](auto p) {
                    constexpr int q = 16 * ch + 2 * p;
                    const float4 t2 = *reinterpret_cast<const float4*>(tp + q);
                    const float4 x2 = *reinterpret_cast<const float4*>(xp + q);
                    v[2 * p] = cfma(v[2 * p], make_float2(t2.x, t2.y), make_float2(x2.x, x2.y));
                    v[2 * p + 1] = cfma(v[2 * p + 1], make_float2(t2.z, t2.w), make_float2(x2.z, x2.w));
                });
            }
        });
        __syncthreads();                                 // the modes are read before the next block overwrites them
        dft<16, 1>(v);
        if (ky0 + c < my) {
            float2* const dst = r + img * (int64_t)H * my;
            const uint32_t o0 = (uint32_t)(n1 * my + ky0 + c), os = (uint32_t)(L * my);
#pragma unroll
            for (int n2 = 0; n2 < 16; ++n2) dst[o0 + os * (uint32_t)n2] = v[n2];
        }
    }
}

// persistent grid: as many workgroups as fit on the device at once, at
// most one per work item
template <typename K, typename... A>
hipError_t launch_cols_short(K kernel, int threads, int64_t nitems, hipStream_t s, A... args) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
    if (e != hipSuccess) return e;
    int64_t n = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    if (n > nitems) n = nitems;
    return launch_kernel(kernel, dim3((unsigned)n), dim3(threads), 0, s, args...);
}

bool cols_short_supported(int log2H, int mx) {
    return log2H >= 6 && log2H <= 9 && (2 * mx) % 16 == 0 && 2 * mx <= short_kept(1 << log2H);
}

}  // namespace

bool cols_pruned_supported(int log2H, int mx, int my) {
    if (mx < 1 || my < 1 || my > 64) return false;
    if (cols_short_supported(log2H, mx)) return true;
    if (log2H < 8 || log2H > 11) return false;
    const int Q = 1 << (log2H - 6);
    return 2 * mx <= kMaxKept && (2 * mx) % Q == 0;
}

hipError_t launch_cols_fwd_pruned(const float2* r, float2* xh, int64_t nimg, int log2H, int mx, int my, float scale,
                                  const float2* tw, hipStream_t s) {
    if (!cols_pruned_supported(log2H, mx, my)) return hipErrorInvalidValue;
    if (cols_short_supported(log2H, mx)) {
        const int nkb = (my + kShortC - 1) / kShortC;
        const int64_t ni = nimg * nkb;
        switch (log2H) {
            case 6: return launch_cols_short(k_cols_fwd_short<4>, 64, ni, s, r, xh, ni, nkb, mx, my, scale, tw);
            case 7: return launch_cols_short(k_cols_fwd_short<8>, 128, ni, s, r, xh, ni, nkb, mx, my, scale, tw);
            case 8: return launch_cols_short(k_cols_fwd_short<16>, 256, ni, s, r, xh, ni, nkb, mx, my, scale, tw);
            default: return launch_cols_short(k_cols_fwd_short<32>, 512, ni, s, r, xh, ni, nkb, mx, my, scale, tw);
        }
    }
    const int nkb = (my + kColC - 1) / kColC;
    const int64_t nb = nimg * nkb;
    if (nb >= INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nb), block(kColThreads);
    switch (log2H) {
        case 8: return launch_kernel(k_cols_fwd_pruned<4>, grid, block, 0, s, r, xh, nkb, mx, my, scale, tw);
        case 9: return launch_kernel(k_cols_fwd_pruned<8>, grid, block, 0, s, r, xh, nkb, mx, my, scale, tw);
        case 10: return launch_kernel(k_cols_fwd_pruned<16>, grid, block, 0, s, r, xh, nkb, mx, my, scale, tw);
        default: return launch_kernel(k_cols_fwd_pruned<32>, grid, block, 0, s, r, xh, nkb, mx, my, scale, tw);
    }
}

hipError_t launch_cols_inv_pruned(const float2* yh, float2* r, int64_t nimg, int log2H, int mx, int my,
                                  const float2* tw, hipStream_t s) {
    if (!cols_pruned_supported(log2H, mx, my)) return hipErrorInvalidValue;
    if (cols_short_supported(log2H, mx)) {
        const int nkb = (my + kShortC - 1) / kShortC;
        const int64_t ni = nimg * nkb;
        switch (log2H) {
            case 6: return launch_cols_short(k_cols_inv_short<4>, 64, ni, s, yh, r, ni, nkb, mx, my, tw);
            case 7: return launch_cols_short(k_cols_inv_short<8>, 128, ni, s, yh, r, ni, nkb, mx, my, tw);
            case 8: return launch_cols_short(k_cols_inv_short<16>, 256, ni, s, yh, r, ni, nkb, mx, my, tw);
            default: return launch_cols_short(k_cols_inv_short<32>, 512, ni, s, yh, r, ni, nkb, mx, my, tw);
        }
    }
    const int nkb = (my + kColC - 1) / kColC;
    const int64_t nb = nimg * nkb;
    if (nb >= INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)nb), block(kColThreads);
    switch (log2H) {
        case 8: return launch_kernel(k_cols_inv_pruned<4>, grid, block, 0, s, yh, r, nkb, mx, my, tw);
        case 9: return launch_kernel(k_cols_inv_pruned<8>, grid, block, 0, s, yh, r, nkb, mx, my, tw);
        case 10: return launch_kernel(k_cols_inv_pruned<16>, grid, block, 0, s, yh, r, nkb, mx, my, tw);
        default: return launch_kernel(k_cols_inv_pruned<32>, grid, block, 0, s, yh, r, nkb, mx, my, tw);
    }
}

}  // namespace fno
