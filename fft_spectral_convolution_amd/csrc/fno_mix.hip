// Per-mode channel mix on the fp32 matrix cores (v_mfma_f32_16x16x4_f32).
//
// For every kept mode m the mix is a complex GEMM (TurboFNO blog, section 2.2:
// the frequency-domain GEMM is a per-mode complex multiply-accumulate,
// (a+bi)(c+di) = (ac-bd) + (ad+bc)i):
//   Y_m[b][o] = sum_i X_m[b][i] * W_m[i][o]
// done as four real products, Yr += Xr Wr - Xi Wi and Yi += Xr Wi + Xi Wr,
// all accumulated in fp32.
//
// Workgroup = 8 waves = one tile of 8 consecutive modes x 32 batch rows x 64
// output channels; wave w owns mode m0 + w, i.e. a 32 x 64 complex result =
// 2 x 4 blocks of 16 x 16, each with a real and an imaginary accumulator.
// The input channels are consumed in chunks of 8 (two MFMA k-steps of 4):
//  * the X chunk of all 8 modes ([32 b][8 i][8 m], one 64-byte run per
//    (b, i)) is staged in LDS as [i][m][b] and shared by the 8 waves;
//  * each wave streams its own W_m rows from global memory straight into the
//    B operand, as float4 pairs (o, o + 1): column block (h, parity) holds
//    o = 32 h + 2 c + parity, c < 16.
// Both are fetched two chunks ahead of their use, with unconditional
// (clamped) loads so the compiler can count outstanding loads exactly.
// Results go back through LDS so that every store instruction of a wave
// writes 1 KiB of consecutive output.  Rows, channels and modes past the ends
// are masked.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMixWaves = 8;           // = modes per tile
constexpr int kMixThreads = 64 * kMixWaves;
constexpr int kMixKC = 8;              // input channels per chunk
constexpr int kMixBRows = 32;          // batch rows per tile (2 MFMA row blocks)
constexpr int kMixOCols = 64;          // output channels per tile (4 MFMA column blocks)

struct Addr {
    int64_t sb, sc, st;
    __device__ __forceinline__ int64_t at(int64_t b, int64_t c, int64_t m) const {
        return b * sb + c * sc + (m >> 3) * st + (m & 7);
    }
};

__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// VEC: every (b, c) run of 8 modes is 16-byte aligned and complete (tiled
// layout), so X is read and Y written as float4; otherwise element-wise.
// NCH > 0: exactly NCH chunks of input channels (unrolled); 0: runtime count.
template <int NCH, bool VEC>
__global__ __launch_bounds__(kMixThreads) void k_mix_mfma(const float2* __restrict__ xh, Addr ax,
                                                          const float2* __restrict__ w, float2* __restrict__ yh,
                                                          Addr ay, int B, int Cin, int Cout, int M, int n_mt,
                                                          int n_bt) {
    constexpr int kAS = kMixBRows + 1;                     // [i][m][b] row stride
    constexpr int kYS = kMixOCols + 1;                     // [b8][m][o] row stride
    constexpr int kAChunk = kMixKC * 8 * kAS;
    __shared__ float2 a_lds[2 * kAChunk];                  // 2 x 16.5 KiB
    __shared__ float2 y_lds[8 * 8 * kYS];                  // 32.5 KiB

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
    const int l16 = lane & 15;               // MFMA row (A) / column (B, C)
    const int lk = lane >> 4;                // MFMA k index within a step (0..3)
    const int nch = NCH > 0 ? NCH : (Cin + kMixKC - 1) / kMixKC;
    const int last = nch - 1;

    // staging role: thread -> (b, i, half of the 8 modes) of a chunk
    const int sbl = tid >> 4;
    const int sil = (tid >> 1) & 7;
    const int shalf = tid & 1;
    const int sb_c = (b0 + sbl < B) ? b0 + sbl : B - 1;
    const int mw_c = m < M ? m : M - 1;

    floatx4 cr[2][4], ci[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            cr[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
            ci[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }

    // X[b0 + sbl][chunk * 8 + sil][m0 + 4 * shalf + q], q < 4.  Clamped
    // indices only feed results that are never stored, except channels past
    // Cin, which are zeroed when the chunk is written to LDS.
    auto load_a = [&](int chunk, float2 (&av)[4]) {
        const int i = chunk * kMixKC + sil;
        const int ic = i < Cin ? i : Cin - 1;
        if constexpr (VEC) {
            const float4* src = reinterpret_cast<const float4*>(xh + ax.at(sb_c, ic, m0 + shalf * 4));
            const float4 v0 = src[0], v1 = src[1];
            av[0] = make_float2(v0.x, v0.y);
            av[1] = make_float2(v0.z, v0.w);
            av[2] = make_float2(v1.x, v1.y);
            av[3] = make_float2(v1.z, v1.w);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int mm = m0 + shalf * 4 + q;
                av[q] = xh[ax.at(sb_c, ic, mm < M ? mm : M - 1)];
            }
        }
    };
    auto store_a = [&](int chunk, const float2 (&av)[4], float2* buf) {
        const bool iok = chunk * kMixKC + sil < Cin;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            buf[(sil * 8 + shalf * 4 + q) * kAS + sbl] = iok ? av[q] : make_float2(0.0f, 0.0f);
    };
    // W pairs for k-step s (channels chunk*8 + 4s + lk), column half h:
    // wv[s][h] = (W[i][o], W[i][o + 1]), o = o0 + 32 h + 2 l16 (Cout is even
    // on this path; columns past Cout are clamped and never stored).
    auto load_w = [&](int chunk, float4 (&wv)[2][2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int i = chunk * kMixKC + 4 * s + lk;
            const int ic = i < Cin ? i : Cin - 1;
            const float2* row = w + ((int64_t)mw_c * Cin + ic) * Cout;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                int o = o0 + 32 * h + 2 * l16;
                o = o < Cout ? o : Cout - 2;
                wv[s][h] = *reinterpret_cast<const float4*>(row + o);
            }
        }
    };
    auto mfma_chunk = [&](const float2* buf, const float4 (&wv)[2][2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float2 a[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) a[rb] = buf[((4 * s + lk) * 8 + wave) * kAS + 16 * rb + l16];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const float4 q = wv[s][cb >> 1];
                    const float wr = (cb & 1) ? q.z : q.x;
                    const float wi = (cb & 1) ? q.w : q.y;
                    cr[rb][cb] = mfma16(a[rb].x, wr, cr[rb][cb]);
                    ci[rb][cb] = mfma16(a[rb].x, wi, ci[rb][cb]);
                }
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const float4 q = wv[s][cb >> 1];
                    const float wr = (cb & 1) ? q.z : q.x;
                    const float wi = (cb & 1) ? q.w : q.y;
                    cr[rb][cb] = mfma16(-a[rb].y, wi, cr[rb][cb]);
                    ci[rb][cb] = mfma16(a[rb].y, wr, ci[rb][cb]);
                }
            }
        }
    };

    // Two register sets alternate, each refilled two chunks ahead right after
    // use; the LDS barriers leave those loads in flight.  LDS buffer k & 1 is
    // rewritten only after every wave passed the barrier of chunk k - 1, i.e.
    // after all reads of chunk k - 2.
    float2 aA[4], aB[4];
    float4 wA[2][2], wB[2][2];
    load_a(0, aA);
    load_w(0, wA);
    load_a(min(1, last), aB);
    load_w(min(1, last), wB);
#pragma unroll
    for (int k = 0; k < nch; k += 2) {
        store_a(k, aA, a_lds);
        load_a(min(k + 2, last), aA);
        lds_barrier();
        mfma_chunk(a_lds, wA);
        load_w(min(k + 2, last), wA);
        if (k + 1 >= nch) break;
        store_a(k + 1, aB, a_lds + kAChunk);
        load_a(min(k + 3, last), aB);
        lds_barrier();
        mfma_chunk(a_lds + kAChunk, wB);
        load_w(min(k + 3, last), wB);
    }

    // C layout of a 16x16 block: lane holds column l16 and, in register r,
    // row 4 * lk + r.  Row block rb adds 16; column block cb = 2 h + parity
    // holds o = 32 h + 2 l16 + parity.  Four rounds of 8 batch rows: round rr
    // holds row block rr / 2 and the lanes with lk / 2 == rr % 2.
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int rb = rr >> 1;
        if ((lk >> 1) == (rr & 1)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int bl = 4 * (lk & 1) + r;    // row within the round
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int ol = 32 * (cb >> 1) + 2 * l16 + (cb & 1);
                    y_lds[(bl * 8 + wave) * kYS + ol] = make_float2(cr[rb][cb][r], ci[rb][cb][r]);
                }
            }
        }
        lds_barrier();
        if constexpr (VEC) {
            // thread -> (b, o, half of the modes): consecutive threads write
            // consecutive 32-byte runs, 2 KiB per wave and instruction pair
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int e = tid + kMixThreads * hh;   // 1024 items = 8 b x 64 o x 2 mode halves
                const int bl = e >> 7;
                const int ol = (e >> 1) & 63;
                const int qh = e & 1;
                const int b = b0 + rr * 8 + bl;
                const int o = o0 + ol;
                if (b < B && o < Cout) {
                    float2 v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = y_lds[(bl * 8 + 4 * qh + q) * kYS + ol];
                    float4* dst = reinterpret_cast<float4*>(yh + ay.at(b, o, m0 + 4 * qh));
                    dst[0] = make_float4(v[0].x, v[0].y, v[1].x, v[1].y);
                    dst[1] = make_float4(v[2].x, v[2].y, v[3].x, v[3].y);
                }
            }
        } else {
            const int bl = tid >> 6;
            const int ol = tid & 63;
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

template <bool VEC>
void launch_mix_variant(dim3 grid, hipStream_t s, const float2* xh, Addr ax, const float2* w, float2* yh, Addr ay,
                        int B, int Cin, int Cout, int M, int n_mt, int n_bt) {
    const int nch = (Cin + kMixKC - 1) / kMixKC;
    switch (nch) {
#define CASE(N)                                                                                                   \
    case N:                                                                                                       \
        hipLaunchKernelGGL((k_mix_mfma<N, VEC>), grid, dim3(kMixThreads), 0, s, xh, ax, w, yh, ay, B, Cin, Cout, \
                           M, n_mt, n_bt);                                                                        \
        break;
        CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
        CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
        default:
            hipLaunchKernelGGL((k_mix_mfma<0, VEC>), grid, dim3(kMixThreads), 0, s, xh, ax, w, yh, ay, B, Cin, Cout,
                               M, n_mt, n_bt);
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

bool mix_mfma_supported(int64_t Cout, const void* w) { return Cout % 2 == 0 && aligned16(w); }

hipError_t launch_mix_mfma(const float2* xh, const SpecLayout& lx, const float2* w, float2* yh, const SpecLayout& ly,
                           int64_t B, int64_t Cin, int64_t Cout, int64_t M, hipStream_t s) {
    if (!mix_mfma_supported(Cout, w)) return hipErrorInvalidValue;
    const int n_mt = (int)((M + 7) / 8);
    const int n_bt = (int)((B + kMixBRows - 1) / kMixBRows);
    const int n_ot = (int)((Cout + kMixOCols - 1) / kMixOCols);
    const Addr ax{lx.sb, lx.sc, lx.st};
    const Addr ay{ly.sb, ly.sc, ly.st};
    const dim3 grid((unsigned)((int64_t)n_mt * n_bt * n_ot));
    // float4 access needs every 8-mode run whole and 16-byte aligned: the
    // tiled layout (runs of exactly 8 in a 256-byte aligned workspace) has it.
    const bool vec = lx.sc == 8 && ly.sc == 8 && lx.st % 2 == 0 && ly.st % 2 == 0 && lx.sb % 2 == 0 &&
                     ly.sb % 2 == 0 && M % 8 == 0 && aligned16(xh) && aligned16(yh);
    if (vec) launch_mix_variant<true>(grid, s, xh, ax, w, yh, ay, (int)B, (int)Cin, (int)Cout, (int)M, n_mt, n_bt);
    else launch_mix_variant<false>(grid, s, xh, ax, w, yh, ay, (int)B, (int)Cin, (int)Cout, (int)M, n_mt, n_bt);
    return hipGetLastError();
}

}  // namespace fno
