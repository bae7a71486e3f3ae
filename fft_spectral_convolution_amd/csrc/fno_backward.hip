// Kernels of the backward pass: gradients of a real loss L through the
// spectral convolution, given g = dL/dout.
//
// With the kept modes m, X = the truncated forward transform of x, G the one
// of g and c_m the complex-to-real weight of the mode's ky (1 for ky = 0 and
// ky = W/2, 2 otherwise; FFT blog, section 2.2: C2R from the N/2+1 half
// spectrum), the chain rule through the per-mode product Y = X W (TurboFNO
// blog, section 2.2) gives
//   dL/dx = the same forward -> mix -> inverse chain applied to g with the
//           conjugate-transposed weight W^H[m][o][i] = conj W[m][i][o]
//           (the C2R weights of the inverse already account for c_m);
//   dL/dRe W + i dL/dIm W = c_m sum_b conj(X[b][i][m]) G[b][o][m].
// The transforms and the mix are the forward pass's kernels; this file adds
// the weight adjoint (a conjugating transpose per mode) and the weight
// gradient (a per-mode contraction over the batch).
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kAdjTile = 32;
constexpr int kAdjThreads = 256;
constexpr int kWgWaves = 8;              // = modes per tile
constexpr int kWgThreads = 64 * kWgWaves;
constexpr int kWgKB = 8;                 // batch rows per chunk (two MFMA k-steps)
constexpr int kWgReduceThreads = 256;

typedef float floatx4 __attribute__((ext_vector_type(4)));

// (b, c, m) -> complex element offset of a truncated spectrum
struct SpecAddr {
    int64_t sb, sc, st;
    __device__ __forceinline__ int64_t at(int64_t b, int64_t c, int64_t m) const {
        return b * sb + c * sc + (m >> 3) * st + (m & 7);
    }
};

// wt[m][o][i] = conj(w[m][i][o]): workgroup (m, tile) moves a 32 x 32 tile of
// one mode, read along o and written along i through LDS.
__global__ __launch_bounds__(kAdjThreads) void k_weight_adjoint(const float2* __restrict__ w, float2* __restrict__ wt,
                                                                int Cin, int Cout, int n_ti, int n_to) {
    __shared__ float2 tile[kAdjTile][kAdjTile + 1];
    const int64_t tiles = (int64_t)n_ti * n_to;
    const int64_t m = blockIdx.x / tiles;
    const int t = (int)(blockIdx.x % tiles);
    const int i0 = (t / n_to) * kAdjTile;
    const int o0 = (t % n_to) * kAdjTile;
    const int tx = threadIdx.x & (kAdjTile - 1);
    const int ty = threadIdx.x / kAdjTile;
    const float2* src = w + m * (int64_t)Cin * Cout;
    for (int r = ty; r < kAdjTile; r += kAdjThreads / kAdjTile) {
        const int i = i0 + r, o = o0 + tx;
        if (i < Cin && o < Cout) tile[r][tx] = src[(int64_t)i * Cout + o];
    }
    __syncthreads();
    float2* dst = wt + m * (int64_t)Cin * Cout;
    for (int r = ty; r < kAdjTile; r += kAdjThreads / kAdjTile) {
        const int o = o0 + r, i = i0 + tx;
        if (i < Cin && o < Cout) {
            const float2 v = tile[tx][r];
            dst[(int64_t)o * Cin + i] = make_float2(v.x, -v.y);
        }
    }
}

// ---- weight gradient on the fp32 matrix cores -------------------------------
//
// Per kept mode the weight gradient is a complex GEMM over the batch,
//   GW_m[i][o] = c_m sum_b conj(X_m[b][i]) G_m[b][o],
// run as three real GEMMs (3M form of the conjugated product):
//   P1 = Xr^T Gr,  P2 = Xi^T Gi,  P3 = (Xr - Xi)^T (Gr + Gi),
//   Re = P1 + P2,  Im = P3 - P1 + P2.
// Tile = 8 consecutive modes x 16 RI input channels x 16 NCB output
// channels, one workgroup of 8 waves, wave w owning mode m0 + w (RI x NCB
// MFMA blocks of 16 x 16, three accumulators each).  The batch is consumed in
// chunks of 8 rows (two k-steps of 4): the chunk's runs of 8 modes of X and G
// are loaded as float4 (lanes over the four quarters of a run, then channels,
// so a wave reads whole runs) and staged in LDS as one plane per mode, which
// the waves read as MFMA operands.  Chunks run two ahead in registers over
// two LDS buffers (one barrier per chunk).  When the tiles are too few for
// the CUs the batch is split into `splits` ranges whose partial sums land in
// a workspace and are added (in a fixed order) by a second kernel.

__device__ __forceinline__ floatx4 mfma16(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Work units: (mode tile, split, input-channel tile, output-channel tile),
// output-channel tile fastest.
struct WgGrid {
    int n_it, n_ot, splits, nch;
};

// LDS planes of one operand chunk with 16 NB channels: element (m, b, c) at
// m * kPlane + b * kC + (c ^ 16 (b & 1)).  The swizzle puts the two batch rows
// a half-wave reads (16 channels each) on different bank halves; the plane
// pad of 4 spreads the staging writes (lanes over mode pairs) over banks.
template <int NB>
struct WgPlanes {
    static constexpr int kC = 16 * NB;
    static constexpr int kPlane = 8 * kC + 4;
    static constexpr int kSize = 8 * kPlane;
    __device__ static __forceinline__ int at(int m, int b, int c) {
        return m * kPlane + b * kC + (NB >= 2 ? (c ^ ((b & 1) << 4)) : c);
    }
};

// Load one operand's chunk (8 batch rows from b0, 16 NB channels from c0, the
// tile's 8 modes): thread e = tid + 512 j holds quarter q = e % 4 (modes
// 2q, 2q + 1) of run (b, c).  Indices past the ends are clamped (rows past B
// are zeroed at staging; channels and modes past the ends only feed results
// that are never stored).
template <int NB, bool VEC>
__device__ __forceinline__ void wg_load(const float2* __restrict__ src, const SpecAddr& a, int b0, int B, int c0,
                                        int C, int m0, int M, float4 (&v)[NB]) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int e = (int)threadIdx.x + kWgThreads * j;
        const int q = e & 3;
        const int cl = (e >> 2) % (16 * NB);
        const int bl = (e >> 2) / (16 * NB);
        const int b = b0 + bl < B ? b0 + bl : B - 1;
        const int c = c0 + cl < C ? c0 + cl : C - 1;
        if constexpr (VEC) {
            v[j] = *reinterpret_cast<const float4*>(src + a.at(b, c, m0 + 2 * q));
        } else {
            const int ma = m0 + 2 * q < M ? m0 + 2 * q : M - 1;
            const int mb = m0 + 2 * q + 1 < M ? m0 + 2 * q + 1 : M - 1;
            const float2 u0 = src[a.at(b, c, ma)], u1 = src[a.at(b, c, mb)];
            v[j] = make_float4(u0.x, u0.y, u1.x, u1.y);
        }
    }
}

template <int NB>
__device__ __forceinline__ void wg_store(float2* buf, const float4 (&v)[NB], int b0, int B) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int e = (int)threadIdx.x + kWgThreads * j;
        const int q = e & 3;
        const int cl = (e >> 2) % (16 * NB);
        const int bl = (e >> 2) / (16 * NB);
        const bool ok = b0 + bl < B;
        buf[WgPlanes<NB>::at(2 * q, bl, cl)] = ok ? make_float2(v[j].x, v[j].y) : make_float2(0.0f, 0.0f);
        buf[WgPlanes<NB>::at(2 * q + 1, bl, cl)] = ok ? make_float2(v[j].z, v[j].w) : make_float2(0.0f, 0.0f);
    }
}

// VEC: every 8-mode run whole and 16-byte aligned (float4 access).  With
// splits == 1 the kernel writes c_m GW to gw[m][i][o]; otherwise split s
// writes its unscaled partial to out + s M Cin Cout.
template <int RI, int NCB, bool VEC>
__global__ __launch_bounds__(kWgThreads) void k_weight_grad_mfma(const float2* __restrict__ xh, SpecAddr ax,
                                                                 const float2* __restrict__ gh, SpecAddr ag,
                                                                 float2* __restrict__ out, int B, int Cin, int Cout,
                                                                 int M, int my, int nyq, WgGrid wg) {
    using PX = WgPlanes<RI>;
    using PG = WgPlanes<NCB>;
    __shared__ float2 xs[2 * PX::kSize];
    __shared__ float2 gs[2 * PG::kSize];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lk = lane >> 4;

    // units that share X or G (same mode tile) go to one XCD: under
    // round-robin dispatch the workgroups equal mod 8 share an XCD, and they
    // take one contiguous eighth of the unit sequence
    const int G = gridDim.x;
    const int u = G % 8 == 0 ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int ot = u % wg.n_ot;
    int r = u / wg.n_ot;
    const int it = r % wg.n_it;
    r /= wg.n_it;
    const int sp = r % wg.splits;
    const int m0 = (r / wg.splits) * 8;
    const int i0 = it * 16 * RI;
    const int o0 = ot * 16 * NCB;
    const int k_begin = (int)((int64_t)wg.nch * sp / wg.splits);
    const int k_end = (int)((int64_t)wg.nch * (sp + 1) / wg.splits);
    const int n = k_end - k_begin;

    floatx4 p1[RI][NCB], p2[RI][NCB], p3[RI][NCB];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            p1[ri][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
            p2[ri][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
            p3[ri][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }

    // chunk k of the unit (clamped to its last one: loads are unconditional
    // so that the outstanding-load count is static)
    auto load = [&](int k, float4 (&xv)[RI], float4 (&gv)[NCB]) __attribute__((always_inline)) {
        const int kc = k_begin + (k < n ? k : n - 1);
        wg_load<RI, VEC>(xh, ax, kc * kWgKB, B, i0, Cin, m0, M, xv);
        wg_load<NCB, VEC>(gh, ag, kc * kWgKB, B, o0, Cout, m0, M, gv);
    };
    auto stage = [&](int k, const float4 (&xv)[RI], const float4 (&gv)[NCB], int buf) __attribute__((always_inline)) {
        const int b0 = (k_begin + k) * kWgKB;
        wg_store<RI>(xs + buf * PX::kSize, xv, b0, B);
        wg_store<NCB>(gs + buf * PG::kSize, gv, b0, B);
    };
    auto mfma_chunk = [&](int buf) __attribute__((always_inline)) {
        const float2* xb = xs + buf * PX::kSize;
        const float2* gb = gs + buf * PG::kSize;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int bl = 4 * s + lk;
            float2 a[RI], g[NCB];
#pragma unroll
            for (int ri = 0; ri < RI; ++ri) a[ri] = xb[PX::at(wave, bl, 16 * ri + l16)];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) g[cb] = gb[PG::at(wave, bl, 16 * cb + l16)];
#pragma unroll
            for (int ri = 0; ri < RI; ++ri) {
                const float ad = a[ri].x - a[ri].y;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    p1[ri][cb] = mfma16(a[ri].x, g[cb].x, p1[ri][cb]);
                    p2[ri][cb] = mfma16(a[ri].y, g[cb].y, p2[ri][cb]);
                    p3[ri][cb] = mfma16(ad, g[cb].x + g[cb].y, p3[ri][cb]);
                }
            }
        }
    };

    float4 xA[RI], gA[NCB], xB[RI], gB[NCB];
    load(0, xA, gA);
    load(1, xB, gB);
    // LDS buffer k & 1 is rewritten only after every wave passed the barrier
    // of chunk k - 1, i.e. after all reads of chunk k - 2
    for (int k = 0; k < n; k += 2) {
        stage(k, xA, gA, 0);
        load(k + 2, xA, gA);
        lds_barrier();
        mfma_chunk(0);
        if (k + 1 < n) {                 // uniform
            stage(k + 1, xB, gB, 1);
            load(k + 3, xB, gB);
            lds_barrier();
            mfma_chunk(1);
        }
    }

    // C layout of a 16 x 16 block: lane holds column l16 (o) and, in register
    // j, row 4 lk + j (i)
    const int m = m0 + wave;
    if (m >= M) return;                  // uniform per wave
    float c = 1.0f;
    float2* dst = out + (int64_t)sp * M * Cin * Cout + (int64_t)m * Cin * Cout;
    if (wg.splits == 1) {
        const int ky = m % my;
        c = (ky == 0 || ky == nyq) ? 1.0f : 2.0f;
    }
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int o = o0 + 16 * cb + l16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = i0 + 16 * ri + 4 * lk + j;
                if (i < Cin && o < Cout) {
                    const float pr = p1[ri][cb][j], pi = p2[ri][cb][j];
                    const float2 v = make_float2(c * (pr + pi), c * (p3[ri][cb][j] - pr + pi));
                    // the gradient itself streams out; split partials stay cached for the reduction
                    if (wg.splits == 1) nt_store2(&dst[(int64_t)i * Cout + o], v);
                    else dst[(int64_t)i * Cout + o] = v;
                }
            }
        }
}

// gw[e] = c_m sum_s part[s][e] over the splits, in split order.
__global__ __launch_bounds__(kWgReduceThreads) void k_weight_grad_reduce(const float2* __restrict__ part,
                                                                         float2* __restrict__ gw, int64_t n,
                                                                         int64_t per_mode, int splits, int my,
                                                                         int nyq) {
    const int64_t stride = (int64_t)gridDim.x * kWgReduceThreads;
    for (int64_t e = (int64_t)blockIdx.x * kWgReduceThreads + threadIdx.x; e < n; e += stride) {
        float2 acc = part[e];
        for (int sp = 1; sp < splits; ++sp) acc = cadd(acc, part[(int64_t)sp * n + e]);
        const int ky = (int)((e / per_mode) % my);
        nt_store2(&gw[e], cscale(acc, (ky == 0 || ky == nyq) ? 1.0f : 2.0f));
    }
}

struct WgPlan {
    int ri, ncb;
    WgGrid grid;
    int64_t units;
    size_t ws_bytes;                     // partial sums (splits > 1)
};

WgPlan weight_grad_plan(int64_t B, int64_t Cin, int64_t Cout, int64_t M, int cus) {
    WgPlan p;
    // tile shape: the largest (fewest re-reads of X and G) that still gives
    // every CU a tile, else the smallest, with the batch split below.  The
    // 32 x 32 tiles run two workgroups per CU (66 KiB of LDS each), which
    // overlaps one tile's result writes with another's loads; measured, that
    // beats 32 x 64 tiles (one workgroup per CU) at 128x128 with 64 channels.
    const int ri_max = Cin > 16 ? 2 : 1;
    const int ncb_max = Cout > 16 ? 2 : 1;
    static const int kShapes[3][2] = {{2, 2}, {1, 2}, {1, 1}};
    int64_t tiles = 0;
    for (const auto& sh : kShapes) {
        if (sh[0] > ri_max || sh[1] > ncb_max) continue;
        p.ri = sh[0];
        p.ncb = sh[1];
        p.grid.n_it = (int)((Cin + 16 * p.ri - 1) / (16 * p.ri));
        p.grid.n_ot = (int)((Cout + 16 * p.ncb - 1) / (16 * p.ncb));
        tiles = (M + 7) / 8 * p.grid.n_it * p.grid.n_ot;
        if (tiles >= cus) break;
    }
    p.grid.nch = (int)((B + kWgKB - 1) / kWgKB);
    // split the batch when the tiles leave CUs idle, keeping two chunks per split
    int64_t splits = tiles >= cus ? 1 : (cus + tiles - 1) / tiles;
    const int64_t max_splits = p.grid.nch / 2 > 1 ? p.grid.nch / 2 : 1;
    if (splits > max_splits) splits = max_splits;
    p.grid.splits = (int)splits;
    p.units = tiles * splits;
    p.ws_bytes = splits > 1 ? (size_t)splits * M * Cin * Cout * sizeof(float2) : 0;
    return p;
}

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
    return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int RI, int NCB>
hipError_t launch_wg(bool vec, dim3 grid, hipStream_t s, const float2* xh, SpecAddr ax, const float2* gh,
                     SpecAddr ag, float2* out, int B, int Cin, int Cout, int M, int my, int nyq, WgGrid wg) {
    if (vec)
        return launch_kernel(k_weight_grad_mfma<RI, NCB, true>, grid, dim3(kWgThreads), 0, s, xh, ax, gh, ag, out, B,
                             Cin, Cout, M, my, nyq, wg);
    return launch_kernel(k_weight_grad_mfma<RI, NCB, false>, grid, dim3(kWgThreads), 0, s, xh, ax, gh, ag, out, B,
                         Cin, Cout, M, my, nyq, wg);
}

}  // namespace

hipError_t launch_weight_adjoint(const float2* w, float2* wt, int64_t M, int64_t Cin, int64_t Cout, hipStream_t s) {
    const int64_t n_ti = (Cin + kAdjTile - 1) / kAdjTile;
    const int64_t n_to = (Cout + kAdjTile - 1) / kAdjTile;
    const int64_t nb = M * n_ti * n_to;
    if (nb >= INT32_MAX || Cin > INT32_MAX || Cout > INT32_MAX) return hipErrorInvalidValue;
    return launch_kernel(k_weight_adjoint, dim3((unsigned)nb), dim3(kAdjThreads), 0, s, w, wt, (int)Cin, (int)Cout,
                         (int)n_ti, (int)n_to);
}

size_t weight_grad_workspace(int64_t B, int64_t Cin, int64_t Cout, int64_t M) {
    return weight_grad_plan(B, Cin, Cout, M, device_cus()).ws_bytes;
}

hipError_t launch_weight_grad(const float2* xh, const SpecLayout& lx, const float2* gh, const SpecLayout& lg,
                              float2* gw, int64_t B, int64_t Cin, int64_t Cout, int64_t M, int my, int nyq, void* ws,
                              size_t ws_bytes, int* splits, hipStream_t s) {
    const WgPlan p = weight_grad_plan(B, Cin, Cout, M, device_cus());
    *splits = p.grid.splits;
    if (p.units >= INT32_MAX || B > INT32_MAX || Cin > INT32_MAX || Cout > INT32_MAX || M > INT32_MAX)
        return hipErrorInvalidValue;
    if (p.ws_bytes > ws_bytes || (p.ws_bytes && !ws)) return hipErrorInvalidValue;
    // float4 access needs every 8-mode run whole and 16-byte aligned
    const bool vec = lx.sb % 2 == 0 && lx.sc % 2 == 0 && lx.st % 2 == 0 && lg.sb % 2 == 0 && lg.sc % 2 == 0 &&
                     lg.st % 2 == 0 && M % 8 == 0 && aligned16(xh) && aligned16(gh);
    const SpecAddr ax{lx.sb, lx.sc, lx.st};
    const SpecAddr ag{lg.sb, lg.sc, lg.st};
    float2* out = p.grid.splits > 1 ? static_cast<float2*>(ws) : gw;
    const dim3 grid((unsigned)p.units);
    const int iB = (int)B, iCin = (int)Cin, iCout = (int)Cout, iM = (int)M;
    if (p.ri == 2) return launch_wg<2, 2>(vec, grid, s, xh, ax, gh, ag, out, iB, iCin, iCout, iM, my, nyq, p.grid);
    return p.ncb == 2 ? launch_wg<1, 2>(vec, grid, s, xh, ax, gh, ag, out, iB, iCin, iCout, iM, my, nyq, p.grid)
                      : launch_wg<1, 1>(vec, grid, s, xh, ax, gh, ag, out, iB, iCin, iCout, iM, my, nyq, p.grid);
}

hipError_t launch_weight_grad_reduce(const void* ws, float2* gw, int64_t Cin, int64_t Cout, int64_t M, int splits,
                                     int my, int nyq, hipStream_t s) {
    if (splits < 2 || !ws) return hipErrorInvalidValue;
    const int64_t n = M * Cin * Cout;
    int64_t blocks = (n + kWgReduceThreads - 1) / kWgReduceThreads;
    if (blocks > 8192) blocks = 8192;
    return launch_kernel(k_weight_grad_reduce, dim3((unsigned)blocks), dim3(kWgReduceThreads), 0, s,
                         static_cast<const float2*>(ws), gw, n, Cin * Cout, splits, my, nyq);
}

}  // namespace fno
