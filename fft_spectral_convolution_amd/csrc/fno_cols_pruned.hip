// Pruned column transforms for tall grids (H = 64 Q rows, Q in {4, 8, 16, 32})
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

}  // namespace

bool cols_pruned_supported(int log2H, int mx, int my) {
    if (log2H < 8 || log2H > 11) return false;
    const int Q = 1 << (log2H - 6);
    return mx >= 1 && 2 * mx <= kMaxKept && (2 * mx) % Q == 0 && my >= 1 && my <= 64;
}

hipError_t launch_cols_fwd_pruned(const float2* r, float2* xh, int64_t nimg, int log2H, int mx, int my, float scale,
                                  const float2* tw, hipStream_t s) {
    if (!cols_pruned_supported(log2H, mx, my)) return hipErrorInvalidValue;
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
