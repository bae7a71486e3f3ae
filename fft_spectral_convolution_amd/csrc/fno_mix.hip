// Per-mode channel mix on the fp32 matrix cores (v_mfma_f32_16x16x4_f32).
//
// For every kept mode m the mix is a complex GEMM (TurboFNO blog, section 2.2:
// the frequency-domain GEMM is a per-mode complex multiply-accumulate):
//   Y_m[b][o] = sum_i X_m[b][i] * W_m[i][o].
// It runs as three real GEMMs (the 3M form of the complex product):
//   P1 = Xr Wr,  P2 = Xi Wi,  P3 = (Xr + Xi)(Wr + Wi),
//   Yr = P1 - P2,  Yi = P3 - P1 - P2,
// all accumulated in fp32.
//
// Tile = 8 consecutive modes x 16 RB batch rows x 16 NCB output channels
// (NCB = 4 when Cout allows it, so that each X element is fetched once, else
// 2; RB = 2 unless B is small or the tiles would be too few for the CUs),
// one workgroup of 8 waves; wave w owns mode m0 + w, a 16 RB x 16 NCB result
// = RB x NCB blocks of 16 x 16 with three accumulators each.  Input channels
// are consumed in chunks of 8 (two MFMA k-steps of 4):
//  * the X chunk of all 8 modes ([16 RB b][8 i][8 m], one 64-byte run per
//    (b, i)) is staged in LDS as [i][m][b] and shared by the 8 waves;
//  * each wave streams its own W_m rows from global memory straight into the
//    B operand, as float4 pairs (o, o + 1): column block 2 h + p holds
//    o = 32 h + 2 c + p, c < 16.
// The grid is persistent and every workgroup walks a contiguous range of
// tiles as one flat sequence of chunks: X and W are fetched two chunks ahead
// across tile boundaries (unconditional, clamped loads, so the compiler can count
// outstanding loads exactly), and a tile's results leave through LDS in
// 32-byte runs while the next tile's first chunks are already in flight.
// Rows, channels and modes past the ends are masked.
//
// TW (the adjoint mix of the backward pass): the B operand is the
// conjugate transpose of the stored weight, conj(W_m[o][i]) with W stored
// [m][Cout][Cin] (the forward weight of the layer whose input gradient is
// computed).  Each lane then reads its column's weight row along the
// contraction, as float4 pairs (k, k + 1): within a chunk, k-step s of lane
// group lk contracts channel 2 lk + s (the staged X chunk is read with the
// same order), and column block cb holds o = 16 cb + l16.
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMixWaves = 8;           // = modes per tile
constexpr int kMixThreads = 64 * kMixWaves;
constexpr int kMixKC = 8;              // input channels per chunk

struct Addr {
    int64_t sb, sc, st;
    __device__ __forceinline__ int64_t at(int64_t b, int64_t c, int64_t m) const {
        return b * sb + c * sc + (m >> 3) * st + (m & 7);
    }
};

struct TileGrid {
    int n_mt, n_bt, n_ot, n_tiles;
};

struct Tile {
    int m0, b0, o0;
};

__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// tile t -> (mode tile, batch tile, output tile): output tile fastest, mode
// tile slowest, so that neighbouring tiles share X (same batch rows) or W
// (same modes); KB batch rows and KO output channels per tile
template <int KB, int KO>
__device__ __forceinline__ Tile tile_of(const TileGrid& tg, int t) {
    const int ot = t % tg.n_ot;
    const int r = t / tg.n_ot;
    return Tile{(r / tg.n_bt) * 8, (r % tg.n_bt) * KB, ot * KO};
}

// VEC: every (b, c) run of 8 modes is 16-byte aligned and complete (tiled
// layout), so X is read and Y written as float4; otherwise element-wise.
// NCH: chunks of input channels per tile (even; chunks past Cin are zero).
// NCB: 16-column MFMA blocks per tile (2 or 4); RB: 16-row blocks (1 or 2).
// ONE: the grid has exactly one workgroup per tile; every chunk's X and W
// are fetched at once, staged together, and multiplied after one barrier
// (nothing to pipeline across tiles; one memory round trip instead of one per
// chunk pair).
template <int NCH, bool VEC, int NCB, int RB, bool TW, bool ONE = false>
__global__ __launch_bounds__(kMixThreads) void k_mix_mfma(const float2* __restrict__ xh, Addr ax,
                                                          const float2* __restrict__ w, float2* __restrict__ yh,
                                                          Addr ay, int B, int Cin, int Cout, int M, TileGrid tg) {
    static_assert(NCH % 2 == 0, "chunks alternate between two register sets");
    static_assert(NCB == 2 || NCB == 4, "W runs are one or two float4 per lane");
    static_assert(RB == 1 || RB == 2, "one or two 16-row blocks");
    constexpr int kB = 16 * RB;                            // batch rows per tile
    constexpr int kO = 16 * NCB;                           // output channels per tile
    // X chunk in LDS: (i, m, b) at i * kAI + m * kAM + (b ^ 2 (i >> 1)).  The
    // strides and the swizzle make both the staging writes (lanes over
    // mode halves, channels and two batch rows) and the MFMA operand reads
    // (lanes over 16 batch rows and two channels) hit 32 different bank pairs.
    constexpr int kAM = 34;                                // mode stride (complex)
    constexpr int kAI = 8 * kAM;                           // channel stride: 16 mod 32
    constexpr int kAChunk = kMixKC * kAI;
    constexpr int kYS = kO + 4;                            // [b8][m][o] row stride (16-byte rows, 4 mod 8)
    static_assert(!ONE || (!TW && NCB == 2 && NCH <= 8), "one-shot tiles: forward, 32 columns, <= 64 channels");
    __shared__ float2 a_lds[(ONE ? NCH : 2) * kAChunk];    // 2 (or NCH) x 17 KiB
    __shared__ __attribute__((aligned(16))) float2 y_lds[8 * 8 * kYS];   // 18 or 34 KiB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;               // MFMA row (A) / column (B, C)
    const int lk = lane >> 4;                // MFMA k index within a step (0..3)
    // staging role: thread -> (b, i, half of the 8 modes) of a chunk (threads
    // with sbl >= kB stage nothing)
    const int sbl = tid >> 4;
    const bool stager = RB == 2 || sbl < kB;
    const int sil = (tid >> 1) & 7;
    const int shalf = tid & 1;

    // X[b0 + sbl][chunk * 8 + sil][m0 + 4 * shalf + q], q < 4.  Clamped
    // indices only feed results that are never stored, except channels past
    // Cin, which are zeroed when the chunk is written to LDS.
    // Chunk order: every workgroup walks its channel chunks rotated by an
    // even offset of its own.  In lock-step, all workgroups would read the
    // weight rows of the same chunk (the same offset modulo a mode's 32 KiB
    // at c3) at once; on some devices' memory placements those reads pile
    // onto a subset of the HBM channels (the kernel took 41 us instead of 30
    // on such a device, 30 with the rotation).  The rotation changes only
    // the order of the sum over input channels.
    const int rot = (int)(blockIdx.x % (NCH / 2)) * 2;
    auto load_a = [&](const Tile& tl, int chunk, float2 (&av)[4]) __attribute__((always_inline)) {
        chunk = (chunk + rot) % NCH;
        const int i = chunk * kMixKC + sil;
        const int ic = i < Cin ? i : Cin - 1;
        const int bl = RB == 2 ? sbl : sbl % kB;   // non-stagers repeat a stager's row (same lines)
        const int b = tl.b0 + bl < B ? tl.b0 + bl : B - 1;
        if constexpr (VEC) {
            const float4* src = reinterpret_cast<const float4*>(xh + ax.at(b, ic, tl.m0 + shalf * 4));
            const float4 v0 = src[0], v1 = src[1];
            av[0] = make_float2(v0.x, v0.y);
            av[1] = make_float2(v0.z, v0.w);
            av[2] = make_float2(v1.x, v1.y);
            av[3] = make_float2(v1.z, v1.w);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int mm = tl.m0 + shalf * 4 + q;
                av[q] = xh[ax.at(b, ic, mm < M ? mm : M - 1)];
            }
        }
    };
    auto store_a = [&](int chunk, const float2 (&av)[4], float2* buf) __attribute__((always_inline)) {
        chunk = (chunk + rot) % NCH;
        if (!stager) return;
        const bool iok = chunk * kMixKC + sil < Cin;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            buf[sil * kAI + (shalf * 4 + q) * kAM + (sbl ^ (2 * (sil >> 1)))] = iok ? av[q] : make_float2(0.0f, 0.0f);
    };
    // W pairs for k-step s (channels chunk*8 + 4s + lk): wv[NCB s + 2 h + p]
    // = W[i][o_h + p], o_h = o0 + 32 h + 2 l16 (Cout is even on this path;
    // columns past Cout are clamped and never stored).
    auto load_w = [&](const Tile& tl, int chunk, float2 (&wv)[2 * NCB]) __attribute__((always_inline)) {
        chunk = (chunk + rot) % NCH;
        const int mw = tl.m0 + wave < M ? tl.m0 + wave : M - 1;
        if constexpr (TW) {
            // conj(W[o][k]), k = chunk * 8 + 2 lk + s: one float4 per column
            // block (Cin is even on this path; pairs past it are clamped and
            // meet zeroed X channels)
            int k = chunk * kMixKC + 2 * lk;
            k = k < Cin ? k : Cin - 2;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                int o = tl.o0 + 16 * cb + l16;
                o = o < Cout ? o : Cout - 1;
                const float4 v = *reinterpret_cast<const float4*>(w + ((int64_t)mw * Cout + o) * Cin + k);
                wv[cb] = make_float2(v.x, -v.y);
                wv[NCB + cb] = make_float2(v.z, -v.w);
            }
            return;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int i = chunk * kMixKC + 4 * s + lk;
            const int ic = i < Cin ? i : Cin - 1;
#pragma unroll
            for (int h = 0; h < NCB / 2; ++h) {
                int o = tl.o0 + 32 * h + 2 * l16;
                o = o < Cout ? o : Cout - 2;
                const float4 v = *reinterpret_cast<const float4*>(w + ((int64_t)mw * Cin + ic) * Cout + o);
                wv[NCB * s + 2 * h] = make_float2(v.x, v.y);
                wv[NCB * s + 2 * h + 1] = make_float2(v.z, v.w);
            }
        }
    };

    floatx4 p1[RB][NCB], p2[RB][NCB], p3[RB][NCB];
    auto mfma_chunk = [&](const float2* buf, const float2 (&wv)[2 * NCB]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            float2 a[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int i = TW ? 2 * lk + s : 4 * s + lk;
                a[rb] = buf[i * kAI + wave * kAM + ((16 * rb + l16) ^ (2 * (i >> 1)))];
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float as = a[rb].x + a[rb].y;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const float2 wc = wv[NCB * s + cb];
                    p1[rb][cb] = mfma16(a[rb].x, wc.x, p1[rb][cb]);
                    p2[rb][cb] = mfma16(a[rb].y, wc.y, p2[rb][cb]);
                    p3[rb][cb] = mfma16(as, wc.x + wc.y, p3[rb][cb]);
                }
            }
        }
    };

    // C layout of a 16x16 block: lane holds column l16 and, in register r,
    // row 4 * lk + r.  Row block rb adds 16; column block 2 h + p holds
    // o = 32 h + 2 l16 + p.  Four rounds of 8 batch rows: round rr holds row block
    // rr / 2 and the lanes with lk / 2 == rr % 2.
    auto epilogue = [&](const Tile& tl) __attribute__((always_inline)) {
#pragma unroll
        for (int rr = 0; rr < 2 * RB; ++rr) {
            const int rb = rr >> 1;
            if ((lk >> 1) == (rr & 1)) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int bl = 4 * (lk & 1) + r;    // row within the round
                    // columns 32 h + 2 l16 + p, p < 2, as one 16-byte write per h
                    float yv[2 * NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const float pr = p1[rb][cb][r], pi = p2[rb][cb][r];
                        yv[2 * cb] = pr - pi;
                        yv[2 * cb + 1] = p3[rb][cb][r] - pr - pi;
                    }
                    if constexpr (TW) {
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            y_lds[(bl * 8 + wave) * kYS + 16 * cb + l16] = make_float2(yv[2 * cb], yv[2 * cb + 1]);
                    } else {
#pragma unroll
                        for (int h = 0; h < NCB / 2; ++h)
                            *reinterpret_cast<float4*>(y_lds + (bl * 8 + wave) * kYS + 32 * h + 2 * l16) =
                                make_float4(yv[4 * h], yv[4 * h + 1], yv[4 * h + 2], yv[4 * h + 3]);
                    }
                }
            }
            lds_barrier();
            // item -> (b, o, half of the modes) of the round: consecutive
            // items write consecutive 32-byte runs
#pragma unroll
            for (int it = tid; it < 8 * kO * 2; it += kMixThreads) {
                const int bl_s = it / (2 * kO);
                const int ol_s = (it >> 1) % kO;
                const int qh = it & 1;
                const int b = tl.b0 + rr * 8 + bl_s;
                const int o = tl.o0 + ol_s;
                if (b < B && o < Cout) {
                    float2 v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = y_lds[(bl_s * 8 + 4 * qh + q) * kYS + ol_s];
                    if constexpr (VEC) {
                        float4* dst = reinterpret_cast<float4*>(yh + ay.at(b, o, tl.m0 + 4 * qh));
                        dst[0] = make_float4(v[0].x, v[0].y, v[1].x, v[1].y);
                        dst[1] = make_float4(v[2].x, v[2].y, v[3].x, v[3].y);
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int mm = tl.m0 + 4 * qh + q;
                            if (mm < M) yh[ay.at(b, o, mm)] = v[q];
                        }
                    }
                }
            }
            lds_barrier();
        }
    };

    // Flat chunk sequence over this workgroup's tiles.  Register sets A and B
    // alternate, each refilled two chunks ahead right after use (past the
    // last tile the last chunk is reloaded).  LDS buffer k & 1 is rewritten
    // only after every wave passed the barrier of chunk k - 1, i.e. after all
    // reads of chunk k - 2.
    // Every workgroup walks a contiguous range of the tile sequence.  The
    // ranges are dealt out so that the workgroups of one XCD (indices equal
    // mod 8 under round-robin dispatch) hold one contiguous eighth of the
    // sequence: tiles that share X or W then share that XCD's L2.
    const int G = gridDim.x;
    const int j = G % 8 == 0 ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int t_begin = (int)((int64_t)tg.n_tiles * j / G);
    const int t_end = (int)((int64_t)tg.n_tiles * (j + 1) / G);
    if constexpr (ONE) {
        const Tile one = tile_of<kB, kO>(tg, t_begin);       // t_end == t_begin + 1
        float2 av[NCH][4];
        float2 wv[NCH][2 * NCB];
        static_for<0, NCH>([&](auto c) {
            load_a(one, c, av[c]);
            load_w(one, c, wv[c]);
        });
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                p1[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
                p2[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
                p3[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
        static_for<0, NCH>([&](auto c) { store_a(c, av[c], a_lds + c * kAChunk); });
        lds_barrier();
        static_for<0, NCH>([&](auto c) { mfma_chunk(a_lds + c * kAChunk, wv[c]); });
        epilogue(one);
        return;
    }
    int t = t_begin;
    Tile cur = tile_of<kB, kO>(tg, t);
    Tile nxt = tile_of<kB, kO>(tg, t + 1 < t_end ? t + 1 : t);
    float2 aA[4], aB[4];
    float2 wA[2 * NCB], wB[2 * NCB];
    load_a(cur, 0, aA);
    load_w(cur, 0, wA);
    load_a(cur, 1, aB);
    load_w(cur, 1, wB);
    for (; t < t_end; ++t) {
        const bool more = t + 1 < t_end;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                p1[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
                p2[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
                p3[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int k = 0; k < NCH; k += 2) {
            // chunks k + 2 and k + 3: this tile's, or the next tile's first two
            const bool here = k + 2 < NCH;
            const Tile& t2 = here ? cur : (more ? nxt : cur);
            const int c2 = here ? k + 2 : (more ? 0 : NCH - 1);
            const int c3 = here ? k + 3 : (more ? 1 : NCH - 1);
            store_a(k, aA, a_lds);
            load_a(t2, c2, aA);
            lds_barrier();
            mfma_chunk(a_lds, wA);
            load_w(t2, c2, wA);
            store_a(k + 1, aB, a_lds + kAChunk);
            load_a(t2, c3, aB);
            lds_barrier();
            mfma_chunk(a_lds + kAChunk, wB);
            load_w(t2, c3, wB);
        }
        epilogue(cur);
        cur = nxt;
        nxt = tile_of<kB, kO>(tg, t + 2 < t_end ? t + 2 : (more ? t + 1 : t));
    }
}

template <bool VEC, int NCB, int RB, bool TW = false, bool ONE = false>
hipError_t launch_mix_variant(dim3 grid, hipStream_t s, const float2* xh, Addr ax, const float2* w, float2* yh, Addr ay,
                        int B, int Cin, int Cout, int M, TileGrid tg, int nch) {
#define CASE(N)                                                                                                   \
    case N:                                                                                                       \
        return launch_kernel((k_mix_mfma<N, VEC, NCB, RB, TW, ONE>), grid, dim3(kMixThreads), 0, s, xh, ax, w, yh, ay, B, \
                           Cin, Cout, M, tg);
    if constexpr (ONE) {
        switch (nch) {
            CASE(2) CASE(4) CASE(6) CASE(8)
            default: break;
        }
        return hipErrorInvalidValue;
    }
    switch (nch) {
        CASE(2) CASE(4) CASE(6) CASE(8)
        default: break;
    }
    if constexpr (NCB == 2 && !ONE) {       // the 64-column tiles take at most 8 chunks
        switch (nch) {
            CASE(10) CASE(12) CASE(14) CASE(16)
            default: break;
        }
    }
#undef CASE
    return hipErrorInvalidValue;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Chunks of 8 input channels, rounded up to an even count.
int64_t mix_chunks(int64_t Cin) { return ((Cin + kMixKC - 1) / kMixKC + 1) / 2 * 2; }

// A layout in which the last 8-mode run is whole even when M is not a
// multiple of 8: the tiled one (its tiles always hold 8 modes per channel),
// or a canonical one whose channels are padded to whole runs.  The missing
// modes have slots of their own; the kernel reads those slots and writes
// their results back there (each mode is a separate product, so nothing
// else depends on them).
bool padded_runs(const SpecLayout& l, int64_t M) {
    const int64_t nt = (M + 7) / 8;
    if (l.sc == 8) return l.st >= (int64_t)l.C * 8 && l.sb >= nt * l.st;                    // tiled
    return l.st == 8 && l.sc % 8 == 0 && l.sc >= 8 * nt && l.sb >= (int64_t)l.C * l.sc;   // canonical, padded
}

// float4 access needs every 8-mode run whole and 16-byte aligned: M a
// multiple of 8 or padded_runs (all strides even, 16-byte aligned bases).
bool mix_vec(const float2* xh, const SpecLayout& lx, const float2* yh, const SpecLayout& ly, int64_t M) {
    const bool whole = M % 8 == 0 || (padded_runs(lx, M) && padded_runs(ly, M));
    return lx.sc % 2 == 0 && ly.sc % 2 == 0 && lx.st % 2 == 0 && ly.st % 2 == 0 && lx.sb % 2 == 0 &&
           ly.sb % 2 == 0 && whole && aligned16(xh) && aligned16(yh);
}

}  // namespace

bool mix_mfma_supported(int64_t Cin, int64_t Cout, const void* w) {
    return Cout % 2 == 0 && aligned16(w) && mix_chunks(Cin) <= 16;
}

bool mix_mfma_adjoint_supported(const float2* xh, const SpecLayout& lx, const float2* w, const float2* yh,
                                const SpecLayout& ly, int64_t Cin, int64_t M) {
    return Cin % 2 == 0 && aligned16(w) && mix_chunks(Cin) <= 16 && mix_vec(xh, lx, yh, ly, M);
}

hipError_t launch_mix_mfma(const float2* xh, const SpecLayout& lx, const float2* w, float2* yh, const SpecLayout& ly,
                           int64_t B, int64_t Cin, int64_t Cout, int64_t M, hipStream_t s, bool adjoint) {
    if (adjoint ? !mix_mfma_adjoint_supported(xh, lx, w, yh, ly, Cin, M) : !mix_mfma_supported(Cin, Cout, w))
        return hipErrorInvalidValue;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const bool vec = mix_vec(xh, lx, yh, ly, M);
    const int nch = (int)mix_chunks(Cin);
    // Tile shape: 32 batch rows unless B fits 16 or 32-row tiles would leave
    // CUs without one; 64 output channels when Cout needs more than 32 and
    // the wider tiles still give every CU one (X is then fetched once per
    // mode tile for Cout <= 64), else 32.  The 64-column tiles hold 96
    // accumulators per lane: they are used with float4 access and at most 8
    // channel chunks only, where they fit the registers of two waves per SIMD.
    TileGrid tg;
    tg.n_mt = (int)((M + 7) / 8);
    const bool short_b = B <= 16 || (int64_t)tg.n_mt * ((B + 31) / 32) * ((Cout + 31) / 32) < cus;
    const int b_rows = short_b ? 16 : 32;
    tg.n_bt = (int)((B + b_rows - 1) / b_rows);
    const int64_t mb_tiles = (int64_t)tg.n_mt * tg.n_bt;
    const bool wide = Cout > 32 && vec && nch <= 8 && mb_tiles * ((Cout + 63) / 64) >= cus;
    const int o_cols = wide ? 64 : 32;
    tg.n_ot = (int)((Cout + o_cols - 1) / o_cols);
    const int64_t n_tiles = mb_tiles * tg.n_ot;
    if (n_tiles >= INT32_MAX / 2) return hipErrorInvalidValue;
    tg.n_tiles = (int)n_tiles;
    // one workgroup (8 waves: two per SIMD) per CU, each walking its tiles
    const int64_t g = n_tiles < cus ? n_tiles : cus;
    const Addr ax{lx.sb, lx.sc, lx.st};
    const Addr ay{ly.sb, ly.sc, ly.st};
    const dim3 grid((unsigned)g);
    const int iB = (int)B, iCin = (int)Cin, iCout = (int)Cout, iM = (int)M;
    if (adjoint) {                       // float4 access (vec) on this path
        if (wide && !short_b) return launch_mix_variant<true, 4, 2, true>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
        if (wide) return launch_mix_variant<true, 4, 1, true>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
        if (!short_b) return launch_mix_variant<true, 2, 2, true>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
        return launch_mix_variant<true, 2, 1, true>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    }
    if (wide && !short_b) return launch_mix_variant<true, 4, 2>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    if (wide) return launch_mix_variant<true, 4, 1>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    // one workgroup per tile with 32-column tiles and <= 64 channels: one-shot tiles
    const bool one = n_tiles <= cus && nch <= 8;
    if (vec && !short_b && one)
        return launch_mix_variant<true, 2, 2, false, true>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    if (vec && short_b && one)
        return launch_mix_variant<true, 2, 1, false, true>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    if (vec && !short_b) return launch_mix_variant<true, 2, 2>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    if (vec) return launch_mix_variant<true, 2, 1>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    if (!short_b) return launch_mix_variant<false, 2, 2>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
    return launch_mix_variant<false, 2, 1>(grid, s, xh, ax, w, yh, ay, iB, iCin, iCout, iM, tg, nch);
}

}  // namespace fno
