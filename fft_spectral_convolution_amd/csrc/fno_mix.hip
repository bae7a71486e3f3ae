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
// own W_m rows straight from global memory into the B operand.  Both are
// fetched two chunks ahead of their use.
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
    // X chunks as [i][m][b] (row stride kAS), double-buffered, so the 32 lanes
    // that read one A-operand column touch consecutive addresses; output
    // staging as [b8][m][o] (row stride kYS) for the same reason.
    constexpr int kAS = kMixBRows + 1;
    constexpr int kYS = kMixOCols + 1;
    constexpr int kAChunk = kMixKC * 8 * kAS;
    __shared__ float2 a_lds[2 * kAChunk];                 // 2 x 16.5 KiB
    __shared__ float2 y_lds[8 * 8 * kYS];                 // 32.5 KiB

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
    const int nch = (Cin + kMixKC - 1) / kMixKC;

    // staging role: thread -> (b, i, half of the 8 modes) of a chunk
    const int sbl = tid >> 4;
    const int sil = (tid >> 1) & 7;
    const int shalf = tid & 1;

    floatx16 cr0 = {}, cr1 = {}, ci0 = {}, ci1 = {};

    // All global loads below are unconditional (indices past an end are
    // clamped to a valid element) so that prefetched loads are never waited
    // for early; the only values that must be zero -- X for channels past Cin
    // -- are zeroed when the chunk is written to LDS.  Clamped rows, modes and
    // output channels only feed results that are never stored.
    const int sb_c = (b0 + sbl < B) ? b0 + sbl : B - 1;
    const int mw_c = m_ok ? m : M - 1;
    // X[b0 + sbl][chunk * 8 + sil][m0 + 4 * shalf + q], q < 4
    auto load_a = [&](int chunk, float2 (&av)[4]) {
        const int i = chunk * kMixKC + sil;
        const int ic = i < Cin ? i : Cin - 1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int mm = m0 + shalf * 4 + q;
            av[q] = xh[ax.at(sb_c, ic, mm < M ? mm : M - 1)];
        }
    };
    auto store_a = [&](int chunk, const float2 (&av)[4], float2* buf) {
        const bool iok = chunk * kMixKC + sil < Cin;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            buf[(sil * 8 + shalf * 4 + q) * kAS + sbl] = iok ? av[q] : make_float2(0.0f, 0.0f);
    };
    // W operand for input channel i, output channels o0 + nb*32 + lrow
    auto load_w = [&](int chunk, float2 (&wv)[8]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int i = chunk * kMixKC + 2 * s + lk;
            const int ic = i < Cin ? i : Cin - 1;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int o = o0 + nb * 32 + lrow;
                wv[s * 2 + nb] = w[((int64_t)mw_c * Cin + ic) * Cout + (o < Cout ? o : Cout - 1)];
            }
        }
    };
    auto mfma_chunk = [&](const float2* buf, const float2 (&wv)[8]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float2 a = buf[((2 * s + lk) * 8 + wave) * kAS + lrow];
            const float2 w0 = wv[s * 2 + 0];
            const float2 w1 = wv[s * 2 + 1];
            // four independent accumulators in turn, so no MFMA waits on
            // the result of the one just issued
            cr0 = mfma32(a.x, w0.x, cr0);
            ci0 = mfma32(a.x, w0.y, ci0);
            cr1 = mfma32(a.x, w1.x, cr1);
            ci1 = mfma32(a.x, w1.y, ci1);
            cr0 = mfma32(-a.y, w0.y, cr0);
            ci0 = mfma32(a.y, w0.x, ci0);
            cr1 = mfma32(-a.y, w1.y, cr1);
            ci1 = mfma32(a.y, w1.x, ci1);
        }
    };

    // Two register sets (A chunk + W chunk) alternate, each refilled two
    // chunks ahead right after use; the LDS barriers leave those loads in
    // flight.  LDS buffer k & 1 is rewritten only after every wave passed the
    // barrier of chunk k - 1, i.e. after all reads of chunk k - 2.
    float2 aA[4], aB[4], wA[8], wB[8];
    load_a(0, aA);
    load_w(0, wA);
    if (nch > 1) {
        load_a(1, aB);
        load_w(1, wB);
    }
    for (int k = 0; k < nch; k += 2) {
        store_a(k, aA, a_lds);
        if (k + 2 < nch) load_a(k + 2, aA);
        lds_barrier();
        mfma_chunk(a_lds, wA);
        if (k + 2 < nch) load_w(k + 2, wA);
        if (k + 1 >= nch) break;
        store_a(k + 1, aB, a_lds + kAChunk);
        if (k + 3 < nch) load_a(k + 3, aB);
        lds_barrier();
        mfma_chunk(a_lds + kAChunk, wB);
        if (k + 3 < nch) load_w(k + 3, wB);
    }

    // C layout of the 32x32 block: lane holds column lrow and, in register r,
    // row 8 * (r / 4) + 4 * lk + (r % 4).
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {              // 8 batch rows per round
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = rr * 4 + q;
            const int bl = 4 * lk + q;               // row within the round
            y_lds[(bl * 8 + wave) * kYS + lrow] = make_float2(cr0[r], ci0[r]);
            y_lds[(bl * 8 + wave) * kYS + 32 + lrow] = make_float2(cr1[r], ci1[r]);
        }
        lds_barrier();
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
                    if (mm < M) yh[ay.at(b, o, mm)] = y_lds[(bl * 8 + q) * kYS + ol];
                }
            }
        }
        lds_barrier();
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
