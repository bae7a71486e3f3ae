// Pruned column transforms for tall grids (H = 64 Q rows, Q in {8, 16, 32})
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
// stores touch eight 64-byte runs), runs its Q-point DFT in registers and
// the 64-way sums over n1 go through LDS, 8 kept modes at a time.  The
// twiddles W^{n1 k} of the kept modes are tabulated once per workgroup in LDS
// from the host-built table.  2 mx must be a multiple of Q: then a kept
// mode's residue mod Q is its index's, and every register index is static.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kColThreads = 512;
constexpr int kColC = 8;                 // columns per workgroup
constexpr int kMaxKept = 128;            // 2 mx
constexpr int kRedStride = 64 * 9;       // reduction buffer: [kk][n1] rows of 9 (8 columns + pad)

// Twiddle table T[q][n1] = W^{n1 k_q} for the kept modes k_q (q < 2 mx).
// Every thread issues all of its (at most 16) table reads before it writes
// any entry, so the gathers overlap instead of queueing one by one.
template <int H>
__device__ __forceinline__ void fill_twiddles(float2* T, int mx, const float2* __restrict__ tw, int sign) {
    constexpr int kPer = kMaxKept * 64 / kColThreads;
    const int ne = 2 * mx * 64;
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

template <int Q>
__global__ __launch_bounds__(kColThreads) void k_cols_fwd_pruned(const float2* __restrict__ r,
                                                                 float2* __restrict__ xh, int nkb, int mx, int my,
                                                                 float scale, const float2* __restrict__ tw) {
    constexpr int H = 64 * Q;
    __shared__ float2 T[kMaxKept * 64];              // 64 KiB
    __shared__ float2 red[kColC * kRedStride];       // 36 KiB
    const int tid = threadIdx.x;
    const int c = tid & 7;                           // column within the block
    const int n1 = tid >> 3;                         // row phase
    // column blocks 2j and 2j + 1 (the two halves of every 128-byte line of
    // the row spectrum) go to workgroups on the same XCD at the same time,
    // so that L2 fetches each line once
    const int64_t blk = paired_image(blockIdx.x, (int64_t)gridDim.x);
    const int64_t img = blk / nkb;
    const int ky = (int)(blk % nkb) * kColC + c;
    const bool cok = ky < my;
    const int kyc = cok ? ky : my - 1;

    // column samples n1 + 64 n2 (issued first, so that the twiddle table is
    // built while they are in flight) -> Q-point DFT in registers
    const float2* src = r + img * (int64_t)H * my + kyc;
    float2 v[Q];
#pragma unroll
    for (int n2 = 0; n2 < Q; ++n2) v[n2] = src[(int64_t)(n1 + 64 * n2) * my];
    fill_twiddles<H>(T, mx, tw, -1);
    dft<Q, -1>(v);
    __syncthreads();                                 // twiddle table complete

    float2* const dst = xh + img * (int64_t)(2 * mx) * my;
    const int nk = 2 * mx;
    // reduction role: (kk = wave, column c, eighth p of the 64 phases)
    const int kk_r = tid >> 6;
    const int p_r = (tid >> 3) & 7;
    // kept mode q is k_q = q or H - 2 mx + q; 2 mx is a multiple of Q, so
    // k_q mod Q = q mod Q and every register index below is static
    static_for<0, kMaxKept / 8>([&](auto ch) {
        if (8 * ch < nk) {                           // uniform: chunks of 8 kept modes
            static_for<0, 8>([&](auto kk) {
                constexpr int q = 8 * ch + kk;
                red[kk * kRedStride + n1 * 9 + c] = cmul(T[(q < nk ? q : 0) * 64 + n1], v[q % Q]);
            });
            __syncthreads();
            float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
            for (int t = 0; t < 8; ++t) acc = cadd(acc, red[kk_r * kRedStride + (8 * p_r + t) * 9 + c]);
            // sum over the 8 lanes c + 8 p of the wave
#pragma unroll
            for (int m = 8; m < 64; m <<= 1) {
                acc.x += __shfl_xor(acc.x, m);
                acc.y += __shfl_xor(acc.y, m);
            }
            const int q = 8 * ch + kk_r;
            if (p_r == 0 && cok && q < nk) dst[(int64_t)q * my + ky] = cscale(acc, scale);
            __syncthreads();
        }
    });
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
    const int64_t img = blockIdx.x / nkb;
    const int ky0 = (blockIdx.x % nkb) * kColC;
    const int ky = ky0 + c;
    const int nk = 2 * mx;

    fill_twiddles<H>(T, mx, tw, 1);
    const float2* src = yh + img * (int64_t)nk * my;
    for (int e = tid; e < nk * kColC; e += kColThreads) {
        const int q = e >> 3, cc = e & 7;
        xs[e] = ky0 + cc < my ? src[(int64_t)q * my + ky0 + cc] : make_float2(0.0f, 0.0f);
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
    if (log2H < 9 || log2H > 11) return false;
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
        case 9: return launch_kernel(k_cols_inv_pruned<8>, grid, block, 0, s, yh, r, nkb, mx, my, tw);
        case 10: return launch_kernel(k_cols_inv_pruned<16>, grid, block, 0, s, yh, r, nkb, mx, my, tw);
        default: return launch_kernel(k_cols_inv_pruned<32>, grid, block, 0, s, yh, r, nkb, mx, my, tw);
    }
}

}  // namespace fno
