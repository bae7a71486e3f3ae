// Pruned transforms of real rows of 64 to 4096 points
// when only the bins k < my <= 64 are kept: the forward R2C that computes
// just those bins, and the C2R that rebuilds a row from them (FFT blog,
// section 2.2: R2C / C2R on the N/2+1 half spectrum; TurboFNO blog, section
// 2.1: only the kept modes are ever needed, so the rest is never computed).
//
// One wave per row, lane n1 < 64 holding the samples n = n1 + 64 n2, n2 < Q:
// every load / store instruction of the wave touches 256 consecutive bytes.
// With n = n1 + 64 n2 and W = exp(-2 pi i / N):
//   X[k] = sum_n1 W^{n1 k} Y_n1[k mod Q],   Y_n1 = DFT_Q of lane n1's samples.
// Forward: each lane runs its Q-point real DFT in registers (packed as a
// Q/2-point complex one) and writes its untwiddled residues Y_n1[r] to a
// per-wave LDS stage; the twiddles are applied on the reading side, where
// lane (bin k, quarter q) sums its 16 lanes n1 = 16 q + t as
// W^{16 q k} sum_t (W^k)^t Y_n1 with a binary tree (factors W^k, W^{2k},
// W^{4k}, W^{8k}), and the quarters are added across neighbouring lanes.
// The reading lane needs two twiddles per 16 bins instead of the writing
// lane needing one per bin, which leaves the registers for four waves per
// SIMD at N = 2048.
// Inverse: lane n1 forms V[r] = sum_{k = r mod Q} c_k X[k] W^{-n1 k}
// (c_0 = 1 with the DC imaginary part dropped, c_k = 2 otherwise: the
// Hermitian extension of the half spectrum); the real part of its inverse
// DFT over r is exactly the lane's Q output samples, computed as the C2R of
// the Hermitian part H[r] = (V[r] + conj V[-r]) / 2, packed as a Q/2-point
// complex inverse DFT in registers.  Its twiddles split as
// W^{n1 (r + Q j)} = W^{n1 r} W_64^{n1 j}: the residue factors W^{n1 r} sit
// in registers for Q <= 32 and in a per-workgroup LDS table for Q = 64, so
// the factor W^{-n1 r} is applied once per residue after the sum over j.
// The waves of a workgroup share no data; the grid is persistent, each wave
// walking rows.  Rows of 1024 to 4096 points (Q in {16, 32, 64}) take the
// one-row-per-wave kernels; rows of 64 to 512 points take the short-row
// kernels further down, several rows per wave.
#include "fno_device.hpp"
#include "fno_internal.hpp"
#include "fno_realbins.hpp"

namespace fno {
namespace {

constexpr int kPrunedThreads = 256;     // 4 independent waves
constexpr int kPrunedWaves = kPrunedThreads / 64;
constexpr int kStageStride = 68;        // forward reduction stage row stride (complex)

// index of (bin kk, lane n1) in a wave's forward reduction stage
__device__ __forceinline__ int stage_at(int kk, int n1) { return kk * kStageStride + n1 + (n1 >> 4); }


// Residue-factored twiddles of a row of N = 64 Q points, lane n1:
// W^{n1 k} = res(k mod Q) * W_64^{n1 (k div Q)} (W = exp(-2 pi i / N)).
// HALF keeps only the residues r <= Q/2 in registers and forms the others as
// W^{n1 r} = W_64^{n1} conj(W^{n1 (Q - r)}) (W^{n1 Q} = W_64^{n1}): one more
// complex product each, Q/2 - 1 fewer register pairs.
template <int Q, bool HALF = false>
struct LaneTwiddles {
    static constexpr int NR = Q <= 32 ? (HALF ? Q / 2 + 1 : Q) : 1;   // residue factors in registers
    static constexpr int NJ = 64 / Q > 1 ? 64 / Q : 1;
    float2 tr[NR];                                  // W^{n1 r}, r < NR (Q <= 32)
    float2 pj[NJ];                                  // W_64^{n1 j}, j < 64 / Q
    const float2* tl;                               // Q = 64: LDS table [r][64 lanes]

    // The residue factors are stored times rs (a real scale folded into
    // them); the W_64 factors are not.
    __device__ __forceinline__ void init(const float2* __restrict__ tw, int lane, float2* lds_table, float rs) {
        constexpr int N = 64 * Q;
        if constexpr (Q <= 32) {
            (void)lds_table;
#pragma unroll
            for (int r = 0; r < NR; ++r) tr[r] = cscale(tw[(lane * r * (kNMax / N)) & (kNMax - 1)], rs);
        } else {
            // 64 x 64 residue factors, filled by the whole workgroup
            for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) {
                const int r = e >> 6, l = e & 63;
                lds_table[e] = cscale(tw[(l * r * (kNMax / N)) & (kNMax - 1)], rs);
            }
            tl = lds_table;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) pj[j] = tw[(lane * j * (kNMax / 64)) & (kNMax - 1)];
        // keep them opaque: formed once here, never re-derived in the row loop
#pragma unroll
        for (int r = 0; r < NR; ++r) asm volatile("" : "+v"(tr[r].x), "+v"(tr[r].y));
    }
    // Hides the factors from loop-invariant code motion (called once per row),
    // so that the derived factors are formed per row, not hoisted into
    // registers.
    __device__ __forceinline__ void opaque() {
#pragma unroll
        for (int r = 0; r < NR; ++r) asm volatile("" : "+v"(tr[r].x), "+v"(tr[r].y));
#pragma unroll
        for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(pj[j].x), "+v"(pj[j].y));
    }
    template <int R>
    __device__ __forceinline__ float2 res(int lane) const {
        if constexpr (Q > 32) return tl[R * 64 + lane];
        else if constexpr (R < NR) return tr[R];
        else return cmul(pj[1], conj2(tr[R < NR ? 0 : Q - R]));
    }
};


template <int Q>
__global__ __launch_bounds__(kPrunedThreads) __attribute__((amdgpu_waves_per_eu(Q == 64 ? 2 : 4))) void k_rows_fwd_pruned(
    const float* __restrict__ x, float2* __restrict__ y, int64_t nrows, int my, int y_ld, float scale,
    const float2* __restrict__ tw) {
    static_assert(Q == 16 || Q == 32 || Q == 64, "rows of 1024 to 4096 points");
    constexpr int N = 64 * Q;
    constexpr int NZ = Q / 2;
    // The kept bins k < 64 fall on Q residues k mod Q, NJ = 64 / Q bins each.
    // A chunk stages RPC = 16 residues: stage row rr of chunk ch holds lane
    // n1's Y[RPC ch + rr], untwiddled, and each reading lane forms all NJ
    // bins of its residue from one read of its 16 staged values (BPL = NJ
    // bins per lane).
    constexpr int NJ = 64 / Q;
    constexpr int BPL = NJ;
    constexpr int RPC = 16;
    constexpr int NCHK = Q / RPC;
    // The lane's residues above Q/2 are the conjugates of those below
    // (its samples are real): only rows r <= Q/2 are staged, once per row.
    constexpr int SROWS = NZ + 1;
    __shared__ float2 stage_all[kPrunedWaves][SROWS * kStageStride];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float2* const stage = stage_all[wave];
    // Reduction role: lane (kk_r, q_r) forms the bins k = RPC ch + rr_r +
    // Q (BPL jj_r + b), b < BPL, from lanes n1 = 16 q_r + t, t < 16:
    //   sum_t W^{n1 k} Y_n1[k mod Q] = W^{16 q_r k} sum_t (W^k)^t Y_{16 q_r + t}
    // (the inner sum as a binary tree with factors W^k, W^2k, W^4k, W^8k),
    // and the four quarters q_r are added across neighbouring lanes.
    const int kk_r = lane >> 2;
    const int q_r = lane & 3;
    const int rr_r = kk_r % RPC;
    const int jj_r = kk_r / RPC;
    // W^k and W^{16 q_r k} of the lane's bins in each chunk, the latter times
    // the output scale (halved: the bins below are doubled).  A residue
    // r > Q/2 reads the staged row Q - r, i.e. conj(Y[r]); its factors are
    // conjugated too, so that the tree yields the conjugate of the bin, and
    // the sign of the imaginary part is restored on the store.
    float2 wk[NCHK][BPL], vk[NCHK][BPL];
    const float half_scale = 0.5f * scale;
#pragma unroll
    for (int ch = 0; ch < NCHK; ++ch)
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            const int k = RPC * ch + rr_r + Q * (BPL * jj_r + b);
            const bool cj = RPC * ch + rr_r > NZ;
            const float2 w = tw[(k * (kNMax / N)) & (kNMax - 1)];
            const float2 u = cscale(tw[(16 * q_r * k * (kNMax / N)) & (kNMax - 1)], half_scale);
            wk[ch][b] = cj ? conj2(w) : w;
            vk[ch][b] = cj ? conj2(u) : u;
        }
    // staged row of the lane's residue in chunk ch, and the sign of the
    // stored imaginary part
    auto srow_of = [&](int ch) __attribute__((always_inline)) {
        const int r = RPC * ch + rr_r;
        return stage + (r > NZ ? Q - r : r) * kStageStride + 16 * q_r + q_r;   // = stage_at(row, 16 q_r)
    };

    const int64_t nwaves = (int64_t)gridDim.x * kPrunedWaves;
    for (int64_t row = (int64_t)blockIdx.x * kPrunedWaves + wave; row < nrows; row += nwaves) {
#pragma unroll
        for (int ch = 0; ch < NCHK; ++ch)
#pragma unroll
            for (int b = 0; b < BPL; ++b)
                asm volatile("" : "+v"(wk[ch][b].x), "+v"(wk[ch][b].y), "+v"(vk[ch][b].x), "+v"(vk[ch][b].y));
        const float* src = x + row * N + lane;
        float2 z[NZ];
#pragma unroll
        for (int m = 0; m < NZ; ++m) z[m] = make_float2(src[64 * (2 * m)], src[64 * (2 * m + 1)]);
        dft<NZ, -1>(z);
        // 2 Y[r], r <= Q/2, staged
        static_for<0, SROWS>([&](auto r) { stage[stage_at(r, lane)] = real_bin2<Q, r>(z); });
        wave_lds_sync();

        float2* const dst = y + row * (int64_t)y_ld;
        static_for<0, NCHK>([&](auto ch) {
            if (RPC * ch < my) {                // uniform: chunks with a kept bin
                const float2* const srow = srow_of(ch);
                const bool cj = RPC * ch + rr_r > NZ;
                float2 v[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) v[t] = srow[t];
                // first level of every bin's tree (v is dead after it), then
                // the rest of each tree
                float2 u[BPL][8];
                static_for<0, BPL>([&](auto b) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) u[b][t] = cfma(v[2 * t], wk[ch][b], v[2 * t + 1]);
                });
                static_for<0, BPL>([&](auto b) {
                    if (b == 0 || RPC * ch + Q * b < my) {      // uniform: a kept bin in this group
                        const float2 w2 = cmul(wk[ch][b], wk[ch][b]);
                        const float2 w4 = cmul(w2, w2);
                        const float2 w8 = cmul(w4, w4);
#pragma unroll
                        for (int t = 0; t < 4; ++t) u[b][t] = cfma(u[b][2 * t], w2, u[b][2 * t + 1]);
#pragma unroll
                        for (int t = 0; t < 2; ++t) u[b][t] = cfma(u[b][2 * t], w4, u[b][2 * t + 1]);
                        float2 acc = cmul(vk[ch][b], cfma(u[b][0], w8, u[b][1]));
                        acc = quad_sum(acc);
                        const int k = RPC * ch + rr_r + Q * (BPL * jj_r + b);
                        if (q_r == 0 && k < my) dst[k] = cj ? conj2(acc) : acc;
                    }
                });
            }
        });
        wave_lds_sync();                        // the stage is read before the next row overwrites it
    }
}

// EPI: the fused output epilogue (bias, GELU, second branch) on every
// output, the branch read at the same index.
template <int Q, bool EPI>
__global__ __launch_bounds__(kPrunedThreads) __attribute__((amdgpu_waves_per_eu(EPI ? (Q == 64 ? 3 : 4) : 2))) void k_rows_inv_pruned(const float2* __restrict__ y,
                                                                    float* __restrict__ out, int64_t nrows, int my,
                                                                    int y_ld, float scale,
                                                                    const float2* __restrict__ tw, Epilogue epi) {
    static_assert(Q == 16 || Q == 32 || Q == 64, "rows of 1024 to 4096 points");
    constexpr int N = 64 * Q;
    constexpr int NZ = Q / 2;
    __shared__ float2 xrow_all[kPrunedWaves][64];
    __shared__ float2 table[Q == 64 ? 64 * 64 : 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float2* const xrow = xrow_all[wave];
    // The Hermitian part below is H[r] = (scale / 2) (V[r] + conj V[-r]) with
    // V[r] = sum c_k X[k] ..., c_0 = 1, c_k = 2 otherwise.  With X[0] halved
    // on load every c_k is 2, and the factor 2 (scale / 2) = scale rides on
    // the residue factors.
    LaneTwiddles<Q, true> tws;
    tws.init(tw, lane, table, scale);
    if constexpr (Q == 64) __syncthreads();

    const int64_t nwaves = (int64_t)gridDim.x * kPrunedWaves;
    const int64_t row0 = (int64_t)blockIdx.x * kPrunedWaves + wave;
    // the next row's kept bins are loaded while this row is transformed
    // (the last row of a wave reloads itself)
    auto load_bins = [&](int64_t r) __attribute__((always_inline)) {
        return lane < my ? y[r * (int64_t)y_ld + lane] : make_float2(0.0f, 0.0f);
    };
    float2 vn = row0 < nrows ? load_bins(row0) : make_float2(0.0f, 0.0f);
    for (int64_t row = row0; row < nrows; row += nwaves) {
        if constexpr (Q <= 32) tws.opaque();
        // the row's kept bins, zero past my, DC imaginary part dropped
        {
            float2 v = vn;
            vn = load_bins(row + nwaves < nrows ? row + nwaves : row);
            if (lane == 0) v = make_float2(0.5f * v.x, 0.0f);
            xrow[lane] = v;
        }
        wave_lds_sync();
        // V[r] / 2 = conj(W^{n1 r}) sum_j X'[k] conj(W_64^{n1 j}), k = r + Q j
        // (X' = X with X[0] halved), times scale through the residue factor
        auto vres = [&](auto r) __attribute__((always_inline)) {
            float2 acc = xrow[r];
            static_for<1, 64 / Q>([&](auto j) { acc = cfma(acc, xrow[r + Q * j], conj2(tws.pj[j])); });
            return cmul(acc, conj2(tws.template res<r>(lane)));
        };
        // Hermitian part H[r] = (scale / 2) (V[r] + conj V[-r]), r <= Q/2,
        // each pair V[r], V[Q - r] formed where it is used
        float2 H[NZ + 1];
        static_for<0, NZ + 1>([&](auto r) {
            constexpr int rm = (Q - r) % Q;
            const float2 a = vres(r);
            const float2 b = (rm == r) ? a : vres(std::integral_constant<int, rm>{});
            H[r] = make_float2(a.x + b.x, a.y - b.y);
        });
        wave_lds_sync();                        // the row buffer is read before the next row overwrites it
        float2 z[NZ];
        static_for<0, NZ>([&](auto k) { z[k] = packed_bin<Q, k>(H); });
        dft<NZ, 1>(z);
        float* const dst = out + row * N + lane;
        if constexpr (EPI) {
            // the row's branch through a buffer resource (an empty range for
            // a null branch: its loads read zero, no branch in the code)
            // the row index is uniform across the wave: move it to scalar
            // registers so that the resource and the bias stay scalar
            const uint32_t urow = __builtin_amdgcn_readfirstlane((uint32_t)row);
            const float bias = epi_bias(epi, urow);
            const __amdgpu_buffer_rsrc_t rb =
                make_rsrc(epi.branch ? epi.branch + (int64_t)urow * N : out, epi.branch ? (uint32_t)(N * 4) : 0u);
            // every branch load of the row is issued before the first
            // activation, so that the row waits for one round trip only
            float br[2 * NZ];
#pragma unroll
            for (int k = 0; k < 2 * NZ; ++k) br[k] = buffer_load_f1(rb, (uint32_t)(lane + 64 * k) * 4u, 0);
#pragma unroll
            for (int m = 0; m < NZ; ++m) {
                nt_store(&dst[64 * (2 * m)], epi_apply(epi, z[m].x, bias, br[2 * m]));
                nt_store(&dst[64 * (2 * m + 1)], epi_apply(epi, z[m].y, bias, br[2 * m + 1]));
            }
        } else {
#pragma unroll
            for (int m = 0; m < NZ; ++m) {
                nt_store(&dst[64 * (2 * m)], z[m].x);
                nt_store(&dst[64 * (2 * m + 1)], z[m].y);
            }
        }
    }
}

// ---- short rows: N = 16 L points, L in {4, 8, 16, 32} ------------------------
// One row per wave would leave a lane of a 256-point row four samples, and
// the 64-phase reduction above would cost several times the instructions
// per byte of the long rows.  A row of 64 to 512 points takes L = N / 16
// lanes instead: lane n1 < L holds the samples n1 + L n2 (n2 < 16) and runs
// a 16-point real DFT, and a wave carries 64 / L rows at once.  With
// W = exp(-2 pi i / N):
//   X[k] = sum_{n1 < L} W^{n1 k} Y_n1[k mod 16],
// formed by one reading lane per (row, bin, block of up to 16 phases) with
// the binary tree of the long rows (factors W^k, W^2k, W^4k, ...), the two
// blocks of a 512-point row added across neighbouring lanes.  The inverse
// mirrors the long-row one with 16 residues,
//   V[r] = conj(W^{n1 r}) sum_j X'[r + 16 j] conj(W_L^{n1 j}),
// and carries the same fused epilogue.
template <int L>
__global__ __launch_bounds__(kPrunedThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_rows_fwd_short(
    const float* __restrict__ x, float2* __restrict__ y, int64_t nrows, int my, int y_ld, float scale,
    const float2* __restrict__ tw) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32, "short rows: 64 to 512 points");
    constexpr int Q = 16, N = Q * L, NZ = Q / 2, SROWS = NZ + 1;
    constexpr int RPW = 64 / L;              // rows per wave
    constexpr int PBS = L < 16 ? L : 16;     // phases per block
    constexpr int PB = L / PBS;              // phase blocks per row
    constexpr int SS = L + PB;               // stage row stride (complex): a pad after every block
    constexpr int NSL = RPW * PB;            // slots: every lane holds one item of each
    constexpr int BPS = 64 / NSL;            // bins per slot
    __shared__ float2 stage_all[kPrunedWaves][RPW * SROWS * SS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float2* const stage = stage_all[wave];
    const int rw = lane / L, n1 = lane % L;   // loading role: row rw of the wave's rows, phase n1
    // Reading role: phase block pb and item group g; slot s (bins BPS s ..
    // BPS s + BPS - 1 of every row) holds item s 64/PB + g = (row it mod RPW,
    // bin it div RPW).  A bin whose residue r exceeds Q/2 reads the staged
    // row Q - r (its conjugate) with conjugated factors and conjugates the sum.
    const int pb = lane % PB;
    const int g = lane / PB;
    auto item = [&](int sl, int& rr, int& k) __attribute__((always_inline)) {
        const int it = sl * (64 / PB) + g;
        rr = it % RPW;
        k = it / RPW;
    };
    // W^k of each slot's bin, and W^{PBS pb k} with two blocks per row
    float2 wk[NSL], vk[PB == 2 ? NSL : 1];
    const float half_scale = 0.5f * scale;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
        int rr, k;
        item(sl, rr, k);
        const bool cj = k % Q > NZ;
        const float2 w = tw[(k * (kNMax / N)) & (kNMax - 1)];
        wk[sl] = cj ? conj2(w) : w;
        if constexpr (PB == 2) {
            const float2 u = cscale(tw[(PBS * pb * k * (kNMax / N)) & (kNMax - 1)], half_scale);
            vk[sl] = cj ? conj2(u) : u;
        }
    }
    const int64_t nwaves = (int64_t)gridDim.x * kPrunedWaves;
    for (int64_t row0 = ((int64_t)blockIdx.x * kPrunedWaves + wave) * RPW; row0 < nrows; row0 += nwaves * RPW) {
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) asm volatile("" : "+v"(wk[sl].x), "+v"(wk[sl].y));
        if constexpr (PB == 2) {
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) asm volatile("" : "+v"(vk[sl].x), "+v"(vk[sl].y));
        }
        // a row past the end repeats the last one (never stored)
        const int64_t row = row0 + rw < nrows ? row0 + rw : nrows - 1;
        const float* src = x + row * N + n1;
        float2 z[NZ];
#pragma unroll
        for (int m = 0; m < NZ; ++m) z[m] = make_float2(src[L * (2 * m)], src[L * (2 * m + 1)]);
        dft<NZ, -1>(z);
        // 2 Y[r], r <= Q/2, staged at (row, r, phase n1 + its block's pad)
        static_for<0, SROWS>([&](auto r) { stage[(rw * SROWS + r) * SS + n1 + n1 / PBS] = real_bin2<Q, r>(z); });
        wave_lds_sync();
        static_for<0, NSL>([&](auto sl) {
            if (BPS * sl < my) {                 // uniform: a slot with a kept bin
                int rr, k;
                item(sl, rr, k);
                const int r = k % Q;
                const bool cj = r > NZ;
                const float2* const sp = stage + (rr * SROWS + (cj ? Q - r : r)) * SS + (PBS + 1) * pb;
                // the block's sum over its PBS phases t as a binary tree
                // with the factors W^k, W^2k, W^4k, ...
                float2 v[PBS];
#pragma unroll
                for (int t = 0; t < PBS; ++t) v[t] = sp[t];
                float2 w = wk[sl];
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
                    acc = cscale(v[0], half_scale);
                }
                if (pb == 0 && k < my && row0 + rr < nrows) y[(row0 + rr) * (int64_t)y_ld + k] = cj ? conj2(acc) : acc;
            }
        });
        wave_lds_sync();                        // the stage is read before the next rows overwrite it
    }
}

// NJ: the 16-bin groups that can hold a kept bin (1, 2 or 4: my <= 16 NJ);
// the others are zero and skipped.
template <int L, bool EPI, int NJ>
__global__ __launch_bounds__(kPrunedThreads) __attribute__((amdgpu_waves_per_eu(EPI && L <= 8 ? 3 : 4))) void k_rows_inv_short(
    const float2* __restrict__ y, float* __restrict__ out, int64_t nrows, int my, int y_ld, float scale,
    const float2* __restrict__ tw, Epilogue epi) {
    static_assert(L == 4 || L == 8 || L == 16 || L == 32, "short rows: 64 to 512 points");
    static_assert(NJ == 1 || NJ == 2 || NJ == 4, "16-bin groups");
    constexpr int Q = 16, N = Q * L, NZ = Q / 2;
    constexpr int RPW = 64 / L;
    __shared__ float2 xrow_all[kPrunedWaves][RPW * 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float2* const xrow = xrow_all[wave];
    const int rw = lane / L, n1 = lane % L;
    // residue factors W^{n1 r} (r <= Q/2) times scale (X[0] is halved on load,
    // so every bin counts twice and 2 (scale / 2) = scale), and W^{16 n1 j} =
    // W_L^{n1 j}; W^{n1 r} for r > Q/2 is W_L^{n1} conj(W^{n1 (Q - r)}).
    // Without the epilogue they sit in a per-workgroup LDS table (a row of
    // TF factors per phase n1), which frees their registers for more waves;
    // with it they stay in registers (the table measured slower there).
    constexpr int TF = NZ + 5;                // odd: the phases' rows fall on distinct bank pairs
    __shared__ float2 ftab[EPI ? 1 : L * TF];
    float2 tr[EPI ? NZ + 1 : 1], pj[EPI ? 4 : 1];
    if constexpr (EPI) {
#pragma unroll
        for (int r = 0; r <= NZ; ++r) tr[r] = cscale(tw[(n1 * r * (kNMax / N)) & (kNMax - 1)], scale);
#pragma unroll
        for (int j = 0; j < 4; ++j) pj[j] = tw[(16 * n1 * j * (kNMax / N)) & (kNMax - 1)];   // pj[1] is needed for any NJ
    } else {
        // entry t of phase n: W^{n t} scale for t <= Q/2, W_L^{n (t - Q/2)} above
        for (int e = threadIdx.x; e < L * TF; e += kPrunedThreads) {
            const int nn = e / TF, t = e % TF;
            ftab[e] = t <= NZ ? cscale(tw[(nn * t * (kNMax / N)) & (kNMax - 1)], scale)
                              : tw[(16 * nn * (t - NZ) * (kNMax / N)) & (kNMax - 1)];
        }
        __syncthreads();
    }
    const float2* const ft = ftab + (EPI ? 0 : n1 * TF);
    auto trf = [&](int r) __attribute__((always_inline)) {
        if constexpr (EPI) return tr[r];
        else return ft[r];
    };
    auto pjf = [&](int j) __attribute__((always_inline)) {
        if constexpr (EPI) return pj[j];
        else return ft[NZ + j];
    };
    auto res = [&](auto r) __attribute__((always_inline)) {
        if constexpr (r <= NZ) return trf(r);
        else return cmul(pjf(1), conj2(trf(r <= NZ ? 0 : Q - r)));
    };
    const int64_t nwaves = (int64_t)gridDim.x * kPrunedWaves;
    // The bins 0 .. BW - 1 (BW = 16 NJ) of the wave's rows starting at r0,
    // RPL rows per load instruction (lane: row lane / BW, bin lane mod BW),
    // NL loads per lane; zero past my and past the last row (in-range loads
    // only: row and bin clamped, the zeros selected).  The bins past BW are
    // never read.
    constexpr int BW = 16 * NJ;
    constexpr int RPL = 64 / BW;
    constexpr int NL = RPW > RPL ? RPW / RPL : 1;
    const int lrow = lane / BW, lbin = lane % BW;
    auto load_bins = [&](int64_t r0, float2 (&v)[NL]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int64_t r = r0 + i * RPL + lrow;
            const bool keep = lbin < my && r < nrows && i * RPL + lrow < RPW;
            v[i] = y[(r < nrows ? r : nrows - 1) * (int64_t)y_ld + (lbin < my ? lbin : my - 1)];
            if (!keep) v[i] = make_float2(0.0f, 0.0f);
        }
    };
    const int64_t first = ((int64_t)blockIdx.x * kPrunedWaves + wave) * RPW;
    float2 vn[NL];
    load_bins(first < nrows ? first : 0, vn);
    for (int64_t row0 = first; row0 < nrows; row0 += nwaves * RPW) {
        if constexpr (EPI) {
#pragma unroll
            for (int r = 0; r <= NZ; ++r) asm volatile("" : "+v"(tr[r].x), "+v"(tr[r].y));
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(pj[j].x), "+v"(pj[j].y));
        }
        // this group's bins to LDS (the DC bin halved, its imaginary part
        // dropped); the next group's loaded meanwhile
#pragma unroll
        for (int i = 0; i < NL; ++i)
            if (i * RPL + lrow < RPW)
                xrow[(i * RPL + lrow) * 64 + lbin] = lbin == 0 ? make_float2(0.5f * vn[i].x, 0.0f) : vn[i];
        load_bins(row0 + nwaves * RPW < nrows ? row0 + nwaves * RPW : row0, vn);
        wave_lds_sync();
        const float2* const xr = xrow + rw * 64;
        // V[r] = conj(W^{n1 r}) sum_j X'[r + Q j] conj(W_L^{n1 j}) for every
        // residue, one at a time with the next residue's NJ bins read
        // ahead: left alone the compiler issues all 16 NJ reads at once and
        // holds them in registers
        float2 V[Q], cur[NJ], nxt[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) cur[j] = xr[Q * j];
        static_for<0, Q>([&](auto r) {
            if constexpr (r + 1 < Q) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) nxt[j] = xr[r + 1 + Q * j];
            }
            float2 acc = cur[0];
            static_for<1, NJ>([&](auto j) { acc = cfma(acc, cur[j], conj2(pjf(j))); });
            V[r] = cmul(acc, conj2(res(r)));
            asm volatile("" : "+v"(V[r].x), "+v"(V[r].y) : : "memory");
#pragma unroll
            for (int j = 0; j < NJ; ++j) cur[j] = nxt[j];
        });
        // the Hermitian part H[r] = V[r] + conj V[-r]
        float2 H[NZ + 1];
#pragma unroll
        for (int r = 0; r <= NZ; ++r) {
            const float2 a = V[r], b = V[(Q - r) % Q];
            H[r] = make_float2(a.x + b.x, a.y - b.y);
        }
        wave_lds_sync();                        // the bins are read before the next rows overwrite them
        float2 z[NZ];
        static_for<0, NZ>([&](auto k) { z[k] = packed_bin<Q, k>(H); });
        dft<NZ, 1>(z);
        float* const dst = out + (row0 + rw) * N + n1;
        if constexpr (EPI) {
            // the wave's rows of the branch through one buffer resource whose
            // range ends at the last row (an empty range for a null branch:
            // its loads read zero); the row group's first row is uniform
            // across the wave, so the resource stays scalar
            const uint32_t urow0 = __builtin_amdgcn_readfirstlane((uint32_t)row0);
            const int64_t left = nrows - row0;
            const uint32_t bytes = (uint32_t)((left < RPW ? left : RPW) * N * 4);
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(epi.branch ? epi.branch + (int64_t)urow0 * N : out,
                                                        epi.branch ? bytes : 0u);
            const float bias = epi_bias(epi, urow0 + rw);
            float br[2 * NZ];
#pragma unroll
            for (int k = 0; k < 2 * NZ; ++k) br[k] = buffer_load_f1(rb, (uint32_t)(rw * N + n1 + L * k) * 4u, 0);
            if (row0 + rw < nrows) {
#pragma unroll
                for (int m = 0; m < NZ; ++m) {
                    nt_store(&dst[L * (2 * m)], epi_apply(epi, z[m].x, bias, br[2 * m]));
                    nt_store(&dst[L * (2 * m + 1)], epi_apply(epi, z[m].y, bias, br[2 * m + 1]));
                }
            }
        } else if (row0 + rw < nrows) {
#pragma unroll
            for (int m = 0; m < NZ; ++m) {
                nt_store(&dst[L * (2 * m)], z[m].x);
                nt_store(&dst[L * (2 * m + 1)], z[m].y);
            }
        }
    }
}

template <typename K, typename TI, typename TO, typename... Extra>
hipError_t launch_rows(K kernel, int64_t nrows, hipStream_t s, const TI* in, TO* out, int my, int y_ld, float scale,
                       const float2* tw, Extra... extra) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kPrunedThreads, 0);
    if (e != hipSuccess) return e;
    int64_t g = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    const int64_t need = (nrows + kPrunedWaves - 1) / kPrunedWaves;
    if (g > need) g = need;
    return launch_kernel(kernel, dim3((unsigned)g), dim3(kPrunedThreads), 0, s, in, out, nrows, my, y_ld, scale, tw,
                         extra...);
}

// the short inverse for the 16-bin groups that my reaches
template <int L, bool EPI>
hipError_t launch_rows_inv_short(int64_t nrows, hipStream_t s, const float2* y, float* out, int my, int y_ld,
                                 float scale, const float2* tw, const Epilogue& epi) {
    if (my <= 16) return launch_rows(k_rows_inv_short<L, EPI, 1>, nrows, s, y, out, my, y_ld, scale, tw, epi);
    if (my <= 32 || L == 4)             // 64-point rows keep at most 32 bins
        return launch_rows(k_rows_inv_short<L, EPI, 2>, nrows, s, y, out, my, y_ld, scale, tw, epi);
    if constexpr (L > 4) return launch_rows(k_rows_inv_short<L, EPI, 4>, nrows, s, y, out, my, y_ld, scale, tw, epi);
    return hipErrorInvalidValue;
}

}  // namespace

// at 64 points the kept bins stay below the Nyquist bin 32 (every kept bin
// but the DC one counts twice in the inverse)
bool rows_pruned_supported(int log2W, int my) {
    return log2W >= 6 && log2W <= 12 && my >= 1 && my <= (log2W == 6 ? 32 : 64);
}

hipError_t launch_rows_fwd_pruned(const float* x, float2* y, int64_t nrows, int log2W, int my, int y_ld, float scale,
                                  const float2* tw, hipStream_t s) {
    if (!rows_pruned_supported(log2W, my) || nrows <= 0) return hipErrorInvalidValue;
    switch (log2W) {
        case 6: return launch_rows(k_rows_fwd_short<4>, nrows, s, x, y, my, y_ld, scale, tw);
        case 7: return launch_rows(k_rows_fwd_short<8>, nrows, s, x, y, my, y_ld, scale, tw);
        case 8: return launch_rows(k_rows_fwd_short<16>, nrows, s, x, y, my, y_ld, scale, tw);
        case 9: return launch_rows(k_rows_fwd_short<32>, nrows, s, x, y, my, y_ld, scale, tw);
        case 10: return launch_rows(k_rows_fwd_pruned<16>, nrows, s, x, y, my, y_ld, scale, tw);
        case 11: return launch_rows(k_rows_fwd_pruned<32>, nrows, s, x, y, my, y_ld, scale, tw);
        default: return launch_rows(k_rows_fwd_pruned<64>, nrows, s, x, y, my, y_ld, scale, tw);
    }
}

hipError_t launch_rows_inv_pruned(const float2* y, float* out, int64_t nrows, int log2W, int my, int y_ld,
                                  float scale, const float2* tw, hipStream_t s, const Epilogue& epi) {
    if (!rows_pruned_supported(log2W, my) || nrows <= 0) return hipErrorInvalidValue;
    if (epi.on) {
        switch (log2W) {
            case 6: return launch_rows_inv_short<4, true>(nrows, s, y, out, my, y_ld, scale, tw, epi);
            case 7: return launch_rows_inv_short<8, true>(nrows, s, y, out, my, y_ld, scale, tw, epi);
            case 8: return launch_rows_inv_short<16, true>(nrows, s, y, out, my, y_ld, scale, tw, epi);
            case 9: return launch_rows_inv_short<32, true>(nrows, s, y, out, my, y_ld, scale, tw, epi);
            case 10: return launch_rows(k_rows_inv_pruned<16, true>, nrows, s, y, out, my, y_ld, scale, tw, epi);
            case 11: return launch_rows(k_rows_inv_pruned<32, true>, nrows, s, y, out, my, y_ld, scale, tw, epi);
            default: return launch_rows(k_rows_inv_pruned<64, true>, nrows, s, y, out, my, y_ld, scale, tw, epi);
        }
    }
    switch (log2W) {
        case 6: return launch_rows_inv_short<4, false>(nrows, s, y, out, my, y_ld, scale, tw, epi);
        case 7: return launch_rows_inv_short<8, false>(nrows, s, y, out, my, y_ld, scale, tw, epi);
        case 8: return launch_rows_inv_short<16, false>(nrows, s, y, out, my, y_ld, scale, tw, epi);
        case 9: return launch_rows_inv_short<32, false>(nrows, s, y, out, my, y_ld, scale, tw, epi);
        case 10: return launch_rows(k_rows_inv_pruned<16, false>, nrows, s, y, out, my, y_ld, scale, tw, epi);
        case 11: return launch_rows(k_rows_inv_pruned<32, false>, nrows, s, y, out, my, y_ld, scale, tw, epi);
        default: return launch_rows(k_rows_inv_pruned<64, false>, nrows, s, y, out, my, y_ld, scale, tw, epi);
    }
}

}  // namespace fno
