// C ABI of libfno: argument validation, per-device state (twiddle table and
// internal workspace), and the choice of schedule for each call.
//
// Validation follows the statement of the problem in the TurboFNO blog
// (section 3.3: contiguous input, power-of-two last dimension) and the
// truncation rule of section 2.2 (kx in [0,mx) u [H-mx,H), ky < my, so
// 2*mx <= H and my <= W/2+1 keep the two kx corners disjoint and inside the
// half spectrum).  Everything is checked before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <memory>
#include <mutex>
#include <vector>

#include "../../include/fno.h"
#include "fno_device.hpp"
#include "fno_internal.hpp"

namespace fno {
namespace {

constexpr int kVersion = 100;   // 0.1.0

thread_local int g_last_hip_error = 0;

// One internal workspace per (device, stream).  `use` is held by a call from
// the moment it takes the buffer until its kernels are enqueued, so that a
// second host thread calling on the same stream cannot free or replace the
// buffer in between (a replacement then waits for that stream's work).
struct Workspace {
    void* stream = nullptr;
    void* ptr = nullptr;
    size_t bytes = 0;
    std::mutex use;
};

struct DeviceState {
    bool init = false;
    float2* twiddle = nullptr;     // kNMax entries exp(-2 pi i m / kNMax)
    std::vector<std::unique_ptr<Workspace>> ws;   // internal grow-only workspaces, one per stream
    void* scratch = nullptr;       // this device's address of `scratch` (set by fno_init)
};

// Scratch of fno_spectral_conv2d_noalloc: the truncated spectra of one call
// live in this fixed device array, so that the call allocates nothing.  Each
// device that loads the library holds its own copy until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in): fno_init looks up its device address per device with
// hipGetSymbolAddress and every use goes through that address.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// A call's hold on its stream's workspace (released when the call returns,
// after its kernels are enqueued).
struct WsLease {
    std::unique_lock<std::mutex> lock;
};

std::mutex g_mutex;
// one state per device, never moved (calls on other devices keep pointers)
std::vector<std::unique_ptr<DeviceState>> g_devices;

// Optional per-kernel timing (fno_set_timing_events): kernel k of a call
// launches with events[2k], events[2k + 1] as its start and stop events.
constexpr int kMaxKernels = 16;
struct Recorder {
    void** events = nullptr;
    int n_events = 0;
    int k = 0;
    const char* names[kMaxKernels] = {};
    int count = 0;
    const char* last_names[kMaxKernels] = {};
    int last_count = 0;
};
thread_local Recorder g_rec;
thread_local LaunchEvents g_pending;

void rec_begin() {
    g_rec.k = 0;
    g_rec.count = 0;
    g_pending = LaunchEvents{};
}

// Call right before launching a kernel: hands the launch its event pair.
void rec_kernel(const char* name, hipStream_t) {
    if (g_rec.events && 2 * g_rec.k + 1 < g_rec.n_events) {
        g_pending.start = static_cast<hipEvent_t>(g_rec.events[2 * g_rec.k]);
        g_pending.stop = static_cast<hipEvent_t>(g_rec.events[2 * g_rec.k + 1]);
    }
    if (g_rec.count < kMaxKernels) g_rec.names[g_rec.count++] = name;
    ++g_rec.k;
}

// Call after the last kernel of a call.
int rec_end(hipStream_t, int rc) {
    g_pending = LaunchEvents{};
    if (rc != 0) return rc;
    for (int i = 0; i < g_rec.count; ++i) g_rec.last_names[i] = g_rec.names[i];
    g_rec.last_count = g_rec.count;
    return rc;
}

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    // a launcher that would have had to build a table while the stream is
    // being captured reports this code
    return e == hipErrorStreamCaptureUnsupported ? FNO_ERR_CAPTURE : FNO_ERR_HIP;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

// Transform lengths: powers of two up to 4096, or other 7-smooth lengths
// (2^a 3^b 5^c 7^d) up to 4096 on the mixed-radix stage kernels.
bool length_ok(int n) { return n >= 2 && n <= kNMax && (is_pow2(n) || mixed_supported(n)); }

// Stage launchers by transform length: power-of-two lengths take the
// specialised and generic kernels, the others the mixed-radix ones.
hipError_t rows_fwd_n(const float* x, float2* y, int64_t nrows, int W, int my, int y_ld, float scale,
                      const float2* tw, hipStream_t s) {
    return is_pow2(W) ? launch_rows_fwd(x, y, nrows, ilog2(W), my, y_ld, scale, tw, s)
                      : launch_rows_fwd_mr(x, y, nrows, W, my, y_ld, scale, s);
}
hipError_t rows_inv_n(const float2* y, float* out, int64_t nrows, int W, int my, int y_ld, float scale,
                      const float2* tw, hipStream_t s, const Epilogue& epi = Epilogue{}) {
    return is_pow2(W) ? launch_rows_inv(y, out, nrows, ilog2(W), my, y_ld, scale, tw, s, epi)
                      : launch_rows_inv_mr(y, out, nrows, W, my, y_ld, scale, s, epi);
}
hipError_t cols_fwd_n(const float2* r, float2* xh, int64_t nimg, int H, int mx, int my, float scale,
                      const float2* tw, hipStream_t s) {
    return is_pow2(H) ? launch_cols_fwd(r, xh, nimg, ilog2(H), mx, my, scale, tw, s)
                      : launch_cols_fwd_mr(r, xh, nimg, H, mx, my, scale, s);
}
hipError_t cols_inv_n(const float2* yh, float2* r, int64_t nimg, int H, int mx, int my, const float2* tw,
                      hipStream_t s) {
    return is_pow2(H) ? launch_cols_inv(yh, r, nimg, ilog2(H), mx, my, tw, s)
                      : launch_cols_inv_mr(yh, r, nimg, H, mx, my, s);
}

// C2R Nyquist bin of a length-W transform (none when W is odd)
int nyquist(int W) { return W % 2 == 0 ? W / 2 : -1; }

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

bool overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Per-device twiddle table, built in double precision with the exact integer
// angle index m and rounded once to float.  Building it allocates and copies,
// which a stream under graph capture does not allow: the call then fails with
// FNO_ERR_CAPTURE (fno_init or any eager call builds it beforehand).
int device_state(DeviceState** out, void* stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    std::lock_guard<std::mutex> lock(g_mutex);
    if ((int)g_devices.size() <= dev) g_devices.resize(dev + 1);
    if (!g_devices[dev]) g_devices[dev] = std::make_unique<DeviceState>();
    DeviceState& st = *g_devices[dev];
    if (!st.init) {
        if (stream_capturing(static_cast<hipStream_t>(stream))) return FNO_ERR_CAPTURE;
        std::vector<float2> host(kNMax);
        for (int m = 0; m < kNMax; ++m) {
            const double ang = 2.0 * M_PI * (double)m / (double)kNMax;
            host[m] = make_float2((float)std::cos(ang), (float)(-std::sin(ang)));
        }
        void* d = nullptr;
        e = hipMalloc(&d, sizeof(float2) * kNMax);
        if (e != hipSuccess) return e == hipErrorOutOfMemory ? FNO_ERR_NOMEM : hip_fail(e);
        e = hipMemcpy(d, host.data(), sizeof(float2) * kNMax, hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(d);
            return hip_fail(e);
        }
        st.twiddle = static_cast<float2*>(d);
        st.init = true;
    }
    *out = &st;
    return FNO_OK;
}

// The internal workspace of calls on `stream`: one grow-only buffer per
// (device, stream), so that calls on different streams never share scratch
// (the FFT blog, sections 2.2 and 5.3: plans and their work areas are made
// once and reused across calls).  On return the caller holds `lease` until it
// has enqueued its kernels.  Growing a buffer first waits for the work already
// enqueued on that stream (which may still read the old buffer), then frees
// it; while the stream is being captured nothing is allocated or freed
// (FNO_ERR_CAPTURE).
int internal_workspace(WsLease& lease, DeviceState* st, size_t bytes, void** ws, void* stream) {
    *ws = nullptr;
    if (bytes == 0) return FNO_OK;
    Workspace* slot = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        for (auto& w : st->ws)
            if (w->stream == stream) slot = w.get();
        if (!slot) {
            st->ws.push_back(std::make_unique<Workspace>());
            slot = st->ws.back().get();
            slot->stream = stream;
        }
    }
    lease.lock = std::unique_lock<std::mutex>(slot->use);
    if (slot->bytes < bytes) {
        hipStream_t hs = static_cast<hipStream_t>(stream);
        if (stream_capturing(hs)) return FNO_ERR_CAPTURE;
        if (slot->ptr) {
            // in-flight work on this stream may still read the old buffer
            hipError_t e = hipStreamSynchronize(hs);
            if (e != hipSuccess) return hip_fail(e);
            (void)hipFree(slot->ptr);
            slot->ptr = nullptr;
            slot->bytes = 0;
        }
        void* d = nullptr;
        hipError_t e = hipMalloc(&d, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e == hipErrorOutOfMemory ? FNO_ERR_NOMEM : hip_fail(e);
        }
        slot->ptr = d;
        slot->bytes = bytes;
    }
    *ws = slot->ptr;
    return FNO_OK;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------

int check_dims_2d(int B, int C, int H, int W, int mx, int my) {
    if (B < 1 || C < 1) return FNO_ERR_SHAPE;
    if (!length_ok(H) || !length_ok(W)) return FNO_ERR_SHAPE;
    if (mx < 1 || 2 * mx > H || my < 1 || my > W / 2 + 1) return FNO_ERR_MODES;
    return FNO_OK;
}

int check_dims_1d(int B, int C, int N, int modes) {
    if (B < 1 || C < 1) return FNO_ERR_SHAPE;
    if (!length_ok(N)) return FNO_ERR_SHAPE;
    if (modes < 1 || modes > N / 2 + 1) return FNO_ERR_MODES;
    return FNO_OK;
}

int check_conv(const float* x, const void* w, const float* out, size_t xbytes, size_t wbytes, size_t obytes) {
    if (!x || !w || !out) return FNO_ERR_NULL;
    if (misaligned(x) || misaligned(w) || misaligned(out)) return FNO_ERR_ALIGN;
    if (overlap(x, xbytes, out, obytes) || overlap(w, wbytes, out, obytes)) return FNO_ERR_ALIAS;
    return FNO_OK;
}

Shape2d make2d(int B, int Cin, int Cout, int H, int W, int mx, int my) {
    Shape2d s;
    s.B = B; s.Cin = Cin; s.Cout = Cout; s.H = H; s.W = W; s.mx = mx; s.my = my;
    s.log2H = ilog2(H); s.log2W = ilog2(W);
    return s;
}

// ---------------------------------------------------------------------------
// schedules
// ---------------------------------------------------------------------------

// The channel mix: MFMA when the per-mode GEMM is big enough to fill a
// 32-row x 64-column tile reasonably, VALU otherwise.
bool use_mfma_mix(int64_t B, int64_t Cin, int64_t Cout) { return B >= 8 && Cin >= 8 && Cout >= 16; }

int run_mix(const float2* xh, const SpecLayout& lx, const float2* w, float2* yh, const SpecLayout& ly, int64_t B,
            int64_t Cin, int64_t Cout, int64_t M, hipStream_t st) {
    hipError_t e;
    if (use_mfma_mix(B, Cin, Cout) && mix_mfma_supported(Cin, Cout, w)) {
        rec_kernel("mix_mfma", st);
        e = launch_mix_mfma(xh, lx, w, yh, ly, B, Cin, Cout, M, st);
    } else {
        rec_kernel("mix_valu", st);
        e = launch_mix_valu(xh, lx, w, yh, ly, B, Cin, Cout, M, st);
    }
    return e == hipSuccess ? FNO_OK : hip_fail(e);
}

// zh(b, i, m) = sum_o gh(b, o, m) conj(w[m][i][o]) (the adjoint mix of the
// backward pass, w the forward weight [m][Cz][Cg]): on the matrix cores with
// the weight read transposed where supported, else through an explicit
// conjugate transpose into wt and the plain mix.
int run_mix_adjoint(const float2* gh, const SpecLayout& lg, const float2* w, float2* wt, float2* zh,
                    const SpecLayout& lz, int64_t B, int64_t Cg, int64_t Cz, int64_t M, hipStream_t st) {
    hipError_t e;
    if (use_mfma_mix(B, Cg, Cz) && mix_mfma_adjoint_supported(gh, lg, w, zh, lz, Cg, M)) {
        rec_kernel("mix_mfma_adj", st);
        e = launch_mix_mfma(gh, lg, w, zh, lz, B, Cg, Cz, M, st, true);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    }
    rec_kernel("wadjoint", st);
    e = launch_weight_adjoint(w, wt, M, Cz, Cg, st);
    if (e != hipSuccess) return hip_fail(e);
    return run_mix(gh, lg, wt, zh, lz, B, Cg, Cz, M, st);
}

bool small_path(const Shape2d& s) {
    return is_pow2(s.H) && is_pow2(s.W) && small2d_supported(s.log2H, s.log2W, s.my);
}

// 256- and 512-row grids of 256 or 512 columns (my <= 32, 16 at 512 rows;
// 2 mx a multiple of 16) with enough images: the forward or inverse
// transform of each image in one kernel, the row spectrum in LDS (same
// canonical spectra as the staged kernels).
bool short2d_path(const Shape2d& s) {
    return is_pow2(s.H) && is_pow2(s.W) && short2d_supported(s.log2H, s.log2W, s.mx, s.my);
}

// Staged transforms: rows and columns as separate kernels, the row spectrum R
// (or R') in workspace; spectra in the canonical layout.  fuse: the
// one-kernel transforms where they apply and pay (not in the unfused
// ablation).
int run_forward2d_staged(const Shape2d& s, int64_t C, const float* x, float2* xh, float2* r, const float2* tw,
                         hipStream_t st, bool fuse = true) {
    const float scale = (float)(1.0 / std::sqrt((double)s.H * (double)s.W));
    if (fuse && short2d_path(s) && short2d_pays(s.B * C, s.log2H, s.log2W)) {
        rec_kernel("fwd2d", st);
        const hipError_t e = launch_fwd2d_short(x, xh, s.B * C, s.log2H, s.log2W, s.mx, s.my, scale, tw, st);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    }
    rec_kernel("rows_fwd", st);
    hipError_t e = rows_fwd_n(x, r, s.B * C * s.H, s.W, s.my, s.my, 1.0f, tw, st);
    if (e != hipSuccess) return hip_fail(e);
    rec_kernel("cols_fwd", st);
    e = cols_fwd_n(r, xh, s.B * C, s.H, s.mx, s.my, scale, tw, st);
    if (e != hipSuccess) return hip_fail(e);
    return FNO_OK;
}

// epi: the fused output epilogue (its rows_per_chan is set here)
int run_inverse2d_staged(const Shape2d& s, int64_t C, const float2* yh, float* out, float2* r, const float2* tw,
                         hipStream_t st, const Epilogue& epi = Epilogue{}, bool fuse = true) {
    const float scale = (float)(1.0 / std::sqrt((double)s.H * (double)s.W));
    if (fuse && short2d_path(s) && short2d_pays(s.B * C, s.log2H, s.log2W)) {
        rec_kernel(epi.on ? "inv2d_gelu" : "inv2d", st);
        Epilogue ep = epi;
        ep.rows_per_chan = (uint32_t)s.H;
        const hipError_t e =
            launch_inv2d_short(yh, out, s.B * C, s.log2H, s.log2W, s.mx, s.my, scale, tw, st, ep);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    }
    rec_kernel("cols_inv", st);
    hipError_t e = cols_inv_n(yh, r, s.B * C, s.H, s.mx, s.my, tw, st);
    if (e != hipSuccess) return hip_fail(e);
    rec_kernel(epi.on ? "rows_inv_gelu" : "rows_inv", st);
    Epilogue ep = epi;
    ep.rows_per_chan = (uint32_t)s.H;
    e = rows_inv_n(r, out, s.B * C * s.H, s.W, s.my, s.my, scale, tw, st, ep);
    if (e != hipSuccess) return hip_fail(e);
    return FNO_OK;
}

// Fused per-image transforms (grids up to 128 x 128), any spectrum layout.
int run_forward2d_small(const Shape2d& s, int64_t C, const float* x, float2* xh, const SpecLayout& lay,
                        const float2* tw, hipStream_t st) {
    const float scale = (float)(1.0 / std::sqrt((double)s.H * (double)s.W));
    rec_kernel("fwd2d", st);
    hipError_t e = rowreg2d_supported(s.log2H, s.log2W, s.mx, s.my, lay)
                       ? launch_fwd2d_rowreg(x, xh, lay, s.B * C, s.log2H, s.log2W, s.mx, s.my, tw, st)
                       : launch_fwd2d_small(x, xh, lay, s.B * C, s.log2H, s.log2W, s.mx, s.my, scale, tw, st);
    return e == hipSuccess ? FNO_OK : hip_fail(e);
}

int run_inverse2d_small(const Shape2d& s, int64_t C, const float2* yh, float* out, const SpecLayout& lay,
                        const float2* tw, hipStream_t st, const Epilogue& epi = Epilogue{}) {
    const float scale = (float)(1.0 / std::sqrt((double)s.H * (double)s.W));
    rec_kernel(epi.on ? "inv2d_gelu" : "inv2d", st);
    Epilogue ep = epi;
    ep.rows_per_chan = 1;                       // per-image kernels pass the image index
    hipError_t e = rowreg2d_supported(s.log2H, s.log2W, s.mx, s.my, lay)
                       ? launch_inv2d_rowreg(yh, out, lay, s.B * C, s.log2H, s.log2W, s.mx, s.my, tw, st, ep)
                       : launch_inv2d_small(yh, out, lay, s.B * C, s.log2H, s.log2W, s.mx, s.my, scale, tw, st, ep);
    return e == hipSuccess ? FNO_OK : hip_fail(e);
}

// Unfused: rows_fwd -> cols_fwd -> mix -> cols_inv -> rows_inv, every
// intermediate spectrum in workspace.  Layout: [R or R' (shared)] [xh] [yh].
size_t unfused_ws_2d(const Shape2d& s) {
    const size_t rmax = (size_t)s.B * (size_t)(s.Cin > s.Cout ? s.Cin : s.Cout) * s.H * s.my * sizeof(float2);
    const size_t m = (size_t)2 * s.mx * s.my;
    return align_up(rmax) + align_up((size_t)s.B * s.Cin * m * sizeof(float2)) +
           align_up((size_t)s.B * s.Cout * m * sizeof(float2));
}

// fuse: the one-kernel 256-row transforms where they apply (the default
// schedule); the unfused ablation runs every pass as its own kernel.
int run_unfused_2d(const Shape2d& s, const float* x, const float2* w, float* out, void* ws, const float2* tw,
                   hipStream_t st, const Epilogue& epi = Epilogue{}, bool fuse = false) {
    const int64_t m = (int64_t)2 * s.mx * s.my;
    const size_t rmax = (size_t)s.B * (size_t)(s.Cin > s.Cout ? s.Cin : s.Cout) * s.H * s.my * sizeof(float2);
    char* p = static_cast<char*>(ws);
    float2* r = reinterpret_cast<float2*>(p);
    p += align_up(rmax);
    float2* xh = reinterpret_cast<float2*>(p);
    p += align_up((size_t)s.B * s.Cin * m * sizeof(float2));
    float2* yh = reinterpret_cast<float2*>(p);
    int rc = run_forward2d_staged(s, s.Cin, x, xh, r, tw, st, fuse);
    if (rc) return rc;
    rc = run_mix(xh, canonical_layout(s.Cin, m), w, yh, canonical_layout(s.Cout, m), s.B, s.Cin, s.Cout, m, st);
    if (rc) return rc;
    return run_inverse2d_staged(s, s.Cout, yh, out, r, tw, st, epi, fuse);
}

// Fused (grids up to 128 x 128): fwd2d -> mix -> inv2d, the truncated spectra
// in the tiled layout (64-byte runs of 8 modes).
size_t fused_small_ws_2d(const Shape2d& s) {
    const int64_t m = (int64_t)2 * s.mx * s.my;
    return align_up((size_t)layout_elems(tiled_layout(s.Cin, m), s.B) * sizeof(float2)) +
           align_up((size_t)layout_elems(tiled_layout(s.Cout, m), s.B) * sizeof(float2));
}

int run_fused_small_2d(const Shape2d& s, const float* x, const float2* w, float* out, void* ws, const float2* tw,
                       hipStream_t st, const Epilogue& epi = Epilogue{}) {
    const int64_t m = (int64_t)2 * s.mx * s.my;
    const SpecLayout lx = tiled_layout(s.Cin, m);
    const SpecLayout ly = tiled_layout(s.Cout, m);
    float2* xh = static_cast<float2*>(ws);
    float2* yh = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                           align_up((size_t)layout_elems(lx, s.B) * sizeof(float2)));
    int rc = run_forward2d_small(s, s.Cin, x, xh, lx, tw, st);
    if (rc) return rc;
    rc = run_mix(xh, lx, w, yh, ly, s.B, s.Cin, s.Cout, m, st);
    if (rc) return rc;
    return run_inverse2d_small(s, s.Cout, yh, out, ly, tw, st, epi);
}

size_t unfused_ws_1d(int64_t B, int64_t Cin, int64_t Cout, int modes) {
    return align_up((size_t)B * Cin * modes * sizeof(float2)) + align_up((size_t)B * Cout * modes * sizeof(float2));
}

int run_unfused_1d(int64_t B, int64_t Cin, int64_t Cout, int N, int modes, const float* x, const float2* w,
                   float* out, void* ws, const float2* tw, hipStream_t st, const Epilogue& epi = Epilogue{}) {
    const float scale = (float)(1.0 / std::sqrt((double)N));
    char* p = static_cast<char*>(ws);
    float2* xh = reinterpret_cast<float2*>(p);
    p += align_up((size_t)B * Cin * modes * sizeof(float2));
    float2* yh = reinterpret_cast<float2*>(p);
    rec_kernel("rows_fwd", st);
    hipError_t e = rows_fwd_n(x, xh, B * Cin, N, modes, modes, scale, tw, st);
    if (e != hipSuccess) return hip_fail(e);
    int rc = run_mix(xh, canonical_layout(Cin, modes), w, yh, canonical_layout(Cout, modes), B, Cin, Cout, modes, st);
    if (rc) return rc;
    rec_kernel(epi.on ? "rows_inv_gelu" : "rows_inv", st);
    Epilogue ep = epi;
    ep.rows_per_chan = 1;
    e = rows_inv_n(yh, out, B * Cout, N, modes, modes, scale, tw, st, ep);
    if (e != hipSuccess) return hip_fail(e);
    return FNO_OK;
}

// Small problems (grids of at most 1024 points, at most 8 channels in and out): the
// whole call as one kernel, one workgroup per batch item with its truncated
// spectra in LDS (no workspace is used).
bool one_kernel_path(const Shape2d& s) {
    return small_path(s) && conv2d_small_fused_supported(s.B, s.Cin, s.Cout, s.log2H, s.log2W, s.mx, s.my);
}

// Workspace of the three-kernel small schedule or of the staged one.
size_t staged_ws_2d(const Shape2d& s) { return small_path(s) ? fused_small_ws_2d(s) : unfused_ws_2d(s); }

// Fastest schedule for the shape (epi: with the fused layer tail, which the
// one-kernel schedule does not take); the workspace size follows the schedule.
size_t best_ws_2d(const Shape2d& s, bool epi = false) {
    return !epi && one_kernel_path(s) ? 0 : staged_ws_2d(s);
}

int run_best_2d(const Shape2d& s, const float* x, const float2* w, float* out, void* ws, const float2* tw,
                hipStream_t st, const Epilogue& epi = Epilogue{}) {
    if (!epi.on && one_kernel_path(s)) {
        rec_kernel("conv_fused", st);
        const float scale = (float)(1.0 / std::sqrt((double)s.H * (double)s.W));
        const hipError_t e =
            launch_conv2d_small_fused(x, w, out, s.B, s.Cin, s.Cout, s.log2H, s.log2W, s.mx, s.my, scale, tw, st);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    }
    if (small_path(s)) return run_fused_small_2d(s, x, w, out, ws, tw, st, epi);
    return run_unfused_2d(s, x, w, out, ws, tw, st, epi, true);
}

// Diagonal global filter: forward -> per-(mode, channel) product -> inverse,
// on the operator's fastest transforms and workspace (C channels in and out).
int run_filter_2d(const Shape2d& s, const float* x, const float2* mask, float* out, void* ws, const float2* tw,
                  hipStream_t st) {
    const int64_t m = (int64_t)2 * s.mx * s.my;
    if (small_path(s)) {
        const SpecLayout lay = tiled_layout(s.Cin, m);
        float2* xh = static_cast<float2*>(ws);
        float2* yh = reinterpret_cast<float2*>(static_cast<char*>(ws) +
                                               align_up((size_t)layout_elems(lay, s.B) * sizeof(float2)));
        if (rowreg2d_supported(s.log2H, s.log2W, s.mx, s.my, lay) &&
            (int64_t)m * s.Cin * 8 < (int64_t)kBufferSkip) {
            // the product folded into the forward transform's stores, on the
            // mask transposed channel-major (in the unused xh region)
            rec_kernel("mask_transpose", st);
            hipError_t e = launch_mask_transpose(mask, xh, m, s.Cin, st);
            if (e != hipSuccess) return hip_fail(e);
            rec_kernel("fwd2d_diag", st);
            e = launch_fwd2d_rowreg(x, yh, lay, s.B * s.Cin, s.log2H, s.log2W, s.mx, s.my, tw, st, xh);
            if (e != hipSuccess) return hip_fail(e);
            return run_inverse2d_small(s, s.Cin, yh, out, lay, tw, st);
        }
        int rc = run_forward2d_small(s, s.Cin, x, xh, lay, tw, st);
        if (rc) return rc;
        rec_kernel("mix_diag", st);
        hipError_t e = launch_mix_diag(xh, yh, lay, mask, s.B, s.Cin, m, st);
        if (e != hipSuccess) return hip_fail(e);
        return run_inverse2d_small(s, s.Cin, yh, out, lay, tw, st);
    }
    const size_t rmax = (size_t)s.B * s.Cin * s.H * s.my * sizeof(float2);
    char* p = static_cast<char*>(ws);
    float2* r = reinterpret_cast<float2*>(p);
    p += align_up(rmax);
    float2* xh = reinterpret_cast<float2*>(p);
    p += align_up((size_t)s.B * s.Cin * m * sizeof(float2));
    float2* yh = reinterpret_cast<float2*>(p);
    const SpecLayout lay = canonical_layout(s.Cin, m);
    int rc = run_forward2d_staged(s, s.Cin, x, xh, r, tw, st);
    if (rc) return rc;
    rec_kernel("mix_diag", st);
    hipError_t e = launch_mix_diag(xh, yh, lay, mask, s.B, s.Cin, m, st);
    if (e != hipSuccess) return hip_fail(e);
    return run_inverse2d_staged(s, s.Cin, yh, out, r, tw, st);
}

int filter2d_common(const float* x, const void* mask, float* out, int B, int C, int H, int W, int mx, int my,
                    void* stream) {
    int rc = check_dims_2d(B, C, H, W, mx, my);
    if (rc) return rc;
    const size_t xbytes = (size_t)B * C * H * W * sizeof(float);
    const size_t mbytes = (size_t)2 * mx * my * C * sizeof(float2);
    rc = check_conv(x, mask, out, xbytes, mbytes, xbytes);
    if (rc) return rc;
    const Shape2d s = make2d(B, C, C, H, W, mx, my);
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    rc = internal_workspace(lease, st, staged_ws_2d(s), &ws, stream);
    if (rc) return rc;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    rec_begin();
    return rec_end(hs, run_filter_2d(s, x, static_cast<const float2*>(mask), out, ws, st->twiddle, hs));
}

int filter1d_common(const float* x, const void* mask, float* out, int B, int C, int N, int modes, void* stream) {
    int rc = check_dims_1d(B, C, N, modes);
    if (rc) return rc;
    const size_t xbytes = (size_t)B * C * N * sizeof(float);
    const size_t mbytes = (size_t)modes * C * sizeof(float2);
    rc = check_conv(x, mask, out, xbytes, mbytes, xbytes);
    if (rc) return rc;
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    const size_t hb = align_up((size_t)B * C * modes * sizeof(float2));
    rc = internal_workspace(lease, st, 2 * hb, &ws, stream);
    if (rc) return rc;
    float2* xh = static_cast<float2*>(ws);
    float2* yh = reinterpret_cast<float2*>(static_cast<char*>(ws) + hb);
    const float scale = (float)(1.0 / std::sqrt((double)N));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    auto run = [&]() -> int {
        rec_kernel("rows_fwd", hs);
        hipError_t e = rows_fwd_n(x, xh, (int64_t)B * C, N, modes, modes, scale, st->twiddle, hs);
        if (e != hipSuccess) return hip_fail(e);
        rec_kernel("mix_diag", hs);
        e = launch_mix_diag(xh, yh, canonical_layout(C, modes), static_cast<const float2*>(mask), B, C, modes, hs);
        if (e != hipSuccess) return hip_fail(e);
        rec_kernel("rows_inv", hs);
        e = rows_inv_n(yh, out, (int64_t)B * C, N, modes, modes, scale, st->twiddle, hs);
        if (e != hipSuccess) return hip_fail(e);
        return FNO_OK;
    };
    rec_begin();
    return rec_end(hs, run());
}

// ---------------------------------------------------------------------------
// zero-padded linear convolution
// ---------------------------------------------------------------------------

// Transform length of the padded grid: the smallest even 7-smooth length
// (2^a 3^b 5^c 7^d, a >= 1) that holds the full linear convolution of n
// samples with a k-tap kernel (even, so that full modes cover every kx);
// 0 when the sizes are out of range.
// Padded length of a linear convolution along a row (1D, or the W axis of
// 2D): the smallest even length >= n + k - 1 that a transform takes (up to
// 4096 any supported one, beyond that up to 8192 a 7-smooth one that is not
// a power of two: the long mixed-radix rows).  The 2D column axis takes
// only lengths up to 4096 (checked by the 2D calls).
int linconv_len(int n, int k) {
    if (n < 1 || k < 1) return 0;
    const int64_t need = (int64_t)n + k - 1;
    for (int64_t p = need < 2 ? 2 : need; p <= 2 * kNMax; ++p)
        if (p % 2 == 0 && (p <= kNMax ? length_ok((int)p) : (!is_pow2((int)p) && mixed_row_supported((int)p))))
            return (int)p;
    return 0;
}

int linconv2d_prepare(const float* k, void* wspec, int Cin, int Cout, int H, int W, int kh, int kw, void* stream) {
    const int PH = linconv_len(H, kh), PW = linconv_len(W, kw);
    if (!PH || !PW || PH > kNMax || Cin < 1 || Cout < 1 || (int64_t)Cin * Cout > INT32_MAX) return FNO_ERR_SHAPE;
    if (!k || !wspec) return FNO_ERR_NULL;
    if (misaligned(k) || misaligned(wspec)) return FNO_ERR_ALIGN;
    const int mx = PH / 2, my = PW / 2 + 1;
    const int64_t io = (int64_t)Cin * Cout, M = (int64_t)PH * my;
    const size_t kbytes = (size_t)io * kh * kw * sizeof(float);
    const size_t wbytes = (size_t)M * io * sizeof(float2);
    if (overlap(k, kbytes, wspec, wbytes)) return FNO_ERR_ALIAS;
    // the kernels as Cout * Cin images of one batch item
    const Shape2d s = make2d(1, (int)io, (int)io, PH, PW, mx, my);
    const size_t kp_b = align_up((size_t)io * PH * PW * sizeof(float));
    const size_t kh_b = align_up((size_t)io * M * sizeof(float2));
    const size_t r_b = small_path(s) ? 0 : align_up((size_t)io * PH * my * sizeof(float2));
    DeviceState* st = nullptr;
    WsLease lease;
    int rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    rc = internal_workspace(lease, st, kp_b + kh_b + r_b, &ws, stream);
    if (rc) return rc;
    float* kp = static_cast<float*>(ws);
    float2* khs = reinterpret_cast<float2*>(static_cast<char*>(ws) + kp_b);
    float2* r = reinterpret_cast<float2*>(static_cast<char*>(ws) + kp_b + kh_b);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    auto run = [&]() -> int {
        rec_kernel("pad", hs);
        hipError_t e = launch_pad2d(k, kp, io, kh, kw, PH, PW, hs);
        if (e != hipSuccess) return hip_fail(e);
        const int frc = small_path(s) ? run_forward2d_small(s, io, kp, khs, canonical_layout(io, M), st->twiddle, hs)
                                      : run_forward2d_staged(s, io, kp, khs, r, st->twiddle, hs);
        if (frc) return frc;
        rec_kernel("spec_to_weight", hs);
        e = launch_spec_to_weight(khs, static_cast<float2*>(wspec), M, Cin, Cout,
                                  (float)std::sqrt((double)PH * (double)PW), hs);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    };
    rec_begin();
    return rec_end(hs, run());
}

// The transforms run on the mixed-radix stage kernels for every padded
// length: their row kernels read the unpadded input (the padding reads as
// zero) and write only the crop window, so no padded copy of x or of the
// output is made.
int linconv2d_run(const float* x, const void* wspec, float* out, int B, int Cin, int Cout, int H, int W, int kh,
                  int kw, int ch, int cw, int Ho, int Wo, void* stream) {
    const int PH = linconv_len(H, kh), PW = linconv_len(W, kw);
    if (!PH || !PW || PH > kNMax || B < 1 || Cin < 1 || Cout < 1) return FNO_ERR_SHAPE;
    if (ch < 0 || cw < 0 || Ho < 1 || Wo < 1 || ch + Ho > H + kh - 1 || cw + Wo > W + kw - 1) return FNO_ERR_SHAPE;
    const int mx = PH / 2, my = PW / 2 + 1;
    const int64_t m = (int64_t)PH * my;
    // the spectra in the tiled layout (batch item, 8-mode tile, channel, 8
    // modes): the matrix-core mix reads and writes whole aligned runs, each
    // tile's runs of all channels contiguous
    const SpecLayout lx = tiled_layout(Cin, m), ly = tiled_layout(Cout, m);
    const size_t xbytes = (size_t)B * Cin * H * W * sizeof(float);
    const size_t wbytes = (size_t)m * Cin * Cout * sizeof(float2);
    const size_t obytes = (size_t)B * Cout * Ho * Wo * sizeof(float);
    int rc = check_conv(x, wspec, out, xbytes, wbytes, obytes);
    if (rc) return rc;
    const int64_t cmax = Cin > Cout ? Cin : Cout;
    const size_t r_b = align_up((size_t)B * cmax * PH * my * sizeof(float2));
    const size_t x_b = align_up((size_t)layout_elems(lx, B) * sizeof(float2));
    const size_t y_b = align_up((size_t)layout_elems(ly, B) * sizeof(float2));
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    rc = internal_workspace(lease, st, r_b + x_b + y_b, &ws, stream);
    if (rc) return rc;
    float2* r = static_cast<float2*>(ws);
    float2* xh = reinterpret_cast<float2*>(static_cast<char*>(ws) + r_b);
    float2* yh = reinterpret_cast<float2*>(static_cast<char*>(ws) + r_b + x_b);
    const float scale = (float)(1.0 / std::sqrt((double)PH * (double)PW));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    auto run = [&]() -> int {
        const RowWindow in_win{PH, H, W, 0, 0};
        rec_kernel("rows_fwd", hs);
        hipError_t e = launch_rows_fwd_mr(x, r, (int64_t)B * Cin * PH, PW, my, my, 1.0f, hs, &in_win);
        if (e != hipSuccess) return hip_fail(e);
        rec_kernel("cols_fwd", hs);
        e = launch_cols_fwd_mr(r, xh, (int64_t)B * Cin, PH, mx, my, scale, hs, &lx);
        if (e != hipSuccess) return hip_fail(e);
        const int mrc = run_mix(xh, lx, static_cast<const float2*>(wspec), yh, ly, B, Cin, Cout, m, hs);
        if (mrc) return mrc;
        rec_kernel("cols_inv", hs);
        e = launch_cols_inv_mr(yh, r, (int64_t)B * Cout, PH, mx, my, hs, &ly);
        if (e != hipSuccess) return hip_fail(e);
        const RowWindow out_win{PH, Ho, Wo, ch, cw};
        rec_kernel("rows_inv", hs);
        e = launch_rows_inv_mr(r, out, (int64_t)B * Cout * PH, PW, my, my, scale, hs, Epilogue{}, &out_win);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    };
    rec_begin();
    return rec_end(hs, run());
}

int linconv1d_prepare(const float* k, void* wspec, int Cin, int Cout, int N, int K, void* stream) {
    const int PN = linconv_len(N, K);
    if (!PN || Cin < 1 || Cout < 1 || (int64_t)Cin * Cout > INT32_MAX) return FNO_ERR_SHAPE;
    if (!k || !wspec) return FNO_ERR_NULL;
    if (misaligned(k) || misaligned(wspec)) return FNO_ERR_ALIGN;
    const int modes = PN / 2 + 1;
    const int64_t io = (int64_t)Cin * Cout;
    if (overlap(k, (size_t)io * K * sizeof(float), wspec, (size_t)modes * io * sizeof(float2))) return FNO_ERR_ALIAS;
    const size_t kp_b = align_up((size_t)io * PN * sizeof(float));
    const size_t kh_b = align_up((size_t)io * modes * sizeof(float2));
    DeviceState* st = nullptr;
    WsLease lease;
    int rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    rc = internal_workspace(lease, st, kp_b + kh_b, &ws, stream);
    if (rc) return rc;
    float* kp = static_cast<float*>(ws);
    float2* khs = reinterpret_cast<float2*>(static_cast<char*>(ws) + kp_b);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    auto run = [&]() -> int {
        rec_kernel("pad", hs);
        hipError_t e = launch_pad2d(k, kp, io, 1, K, 1, PN, hs);
        if (e != hipSuccess) return hip_fail(e);
        rec_kernel("rows_fwd", hs);
        e = rows_fwd_n(kp, khs, io, PN, modes, modes, (float)(1.0 / std::sqrt((double)PN)), st->twiddle, hs);
        if (e != hipSuccess) return hip_fail(e);
        rec_kernel("spec_to_weight", hs);
        e = launch_spec_to_weight(khs, static_cast<float2*>(wspec), modes, Cin, Cout, (float)std::sqrt((double)PN), hs);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    };
    rec_begin();
    return rec_end(hs, run());
}

int linconv1d_run(const float* x, const void* wspec, float* out, int B, int Cin, int Cout, int N, int K, int crop,
                  int No, void* stream) {
    const int PN = linconv_len(N, K);
    if (!PN || B < 1 || Cin < 1 || Cout < 1) return FNO_ERR_SHAPE;
    if (crop < 0 || No < 1 || crop + No > N + K - 1) return FNO_ERR_SHAPE;
    const int modes = PN / 2 + 1;
    const size_t xbytes = (size_t)B * Cin * N * sizeof(float);
    const size_t wbytes = (size_t)modes * Cin * Cout * sizeof(float2);
    const size_t obytes = (size_t)B * Cout * No * sizeof(float);
    int rc = check_conv(x, wspec, out, xbytes, wbytes, obytes);
    if (rc) return rc;
    // each channel's spectrum padded to whole 8-mode runs (see the 2D case)
    const int mp = (modes + 7) / 8 * 8;
    const size_t x_b = align_up((size_t)B * Cin * mp * sizeof(float2));
    const size_t y_b = align_up((size_t)B * Cout * mp * sizeof(float2));
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    rc = internal_workspace(lease, st, x_b + y_b, &ws, stream);
    if (rc) return rc;
    float2* xh = static_cast<float2*>(ws);
    float2* yh = reinterpret_cast<float2*>(static_cast<char*>(ws) + x_b);
    const float scale = (float)(1.0 / std::sqrt((double)PN));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    auto run = [&]() -> int {
        const RowWindow in_win{1, 1, N, 0, 0};
        rec_kernel("rows_fwd", hs);
        hipError_t e = launch_rows_fwd_mr(x, xh, (int64_t)B * Cin, PN, modes, mp, scale, hs, &in_win);
        if (e != hipSuccess) return hip_fail(e);
        const int mrc = run_mix(xh, padded_layout(Cin, modes), static_cast<const float2*>(wspec), yh,
                                padded_layout(Cout, modes), B, Cin, Cout, modes, hs);
        if (mrc) return mrc;
        const RowWindow out_win{1, 1, No, 0, crop};
        rec_kernel("rows_inv", hs);
        e = launch_rows_inv_mr(yh, out, (int64_t)B * Cout, PN, modes, mp, scale, hs, Epilogue{}, &out_win);
        return e == hipSuccess ? FNO_OK : hip_fail(e);
    };
    rec_begin();
    return rec_end(hs, run());
}

// Inputs of the fused output epilogue: bias [Cout] (4-byte aligned) and
// branch (the output's shape, 16-byte aligned) are optional; neither may
// overlap the output.
int check_epilogue(const float* bias, const float* branch, const float* out, int Cout, size_t obytes,
                   int branch_after, Epilogue* epi) {
    if (branch_after != 0 && branch_after != 1) return FNO_ERR_SHAPE;
    if ((bias && (reinterpret_cast<uintptr_t>(bias) & 3u)) || (branch && misaligned(branch))) return FNO_ERR_ALIGN;
    if ((bias && overlap(bias, (size_t)Cout * sizeof(float), out, obytes)) ||
        (branch && overlap(branch, obytes, out, obytes)))
        return FNO_ERR_ALIAS;
    epi->on = true;
    epi->bias = bias;
    epi->branch = branch;
    epi->cout = (uint32_t)Cout;
    epi->branch_after = branch_after;
    return FNO_OK;
}

// The state of the current device as fno_init left it, without building
// anything (nullptr when fno_init has not run on this device).
DeviceState* initialised_state() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (dev < 0 || dev >= (int)g_devices.size() || !g_devices[dev]) return nullptr;
    DeviceState* st = g_devices[dev].get();
    return st->init && st->scratch ? st : nullptr;
}

int conv2d_common(const float* x, const void* w, float* out, int B, int Cin, int Cout, int H, int W, int mx,
                  int my, void* user_ws, size_t user_ws_bytes, bool use_user_ws, bool unfused, void* stream,
                  const Epilogue& epi = Epilogue{}) {
    int rc = check_dims_2d(B, Cin, H, W, mx, my);
    if (rc) return rc;
    if (Cout < 1) return FNO_ERR_SHAPE;
    const size_t xbytes = (size_t)B * Cin * H * W * sizeof(float);
    const size_t obytes = (size_t)B * Cout * H * W * sizeof(float);
    const size_t wbytes = (size_t)2 * mx * my * Cin * Cout * sizeof(float2);
    rc = check_conv(x, w, out, xbytes, wbytes, obytes);
    if (rc) return rc;
    const Shape2d s = make2d(B, Cin, Cout, H, W, mx, my);
    const size_t need = unfused ? unfused_ws_2d(s) : best_ws_2d(s, epi.on);
    void* ws = user_ws;
    if (use_user_ws) {
        if (user_ws_bytes < need || (need > 0 && !user_ws)) return FNO_ERR_WORKSPACE;
        if (need > 0 && (reinterpret_cast<uintptr_t>(user_ws) & 255u)) return FNO_ERR_ALIGN;
    }
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    if (!use_user_ws) {
        rc = internal_workspace(lease, st, need, &ws, stream);
        if (rc) return rc;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const float2* wc = static_cast<const float2*>(w);
    rec_begin();
    if (unfused) return rec_end(hs, run_unfused_2d(s, x, wc, out, ws, st->twiddle, hs, epi));
    return rec_end(hs, run_best_2d(s, x, wc, out, ws, st->twiddle, hs, epi));
}

int conv1d_common(const float* x, const void* w, float* out, int B, int Cin, int Cout, int N, int modes,
                  void* user_ws, size_t user_ws_bytes, bool use_user_ws, bool unfused, void* stream,
                  const Epilogue& epi = Epilogue{}) {
    (void)unfused;
    int rc = check_dims_1d(B, Cin, N, modes);
    if (rc) return rc;
    if (Cout < 1) return FNO_ERR_SHAPE;
    const size_t xbytes = (size_t)B * Cin * N * sizeof(float);
    const size_t obytes = (size_t)B * Cout * N * sizeof(float);
    const size_t wbytes = (size_t)modes * Cin * Cout * sizeof(float2);
    rc = check_conv(x, w, out, xbytes, wbytes, obytes);
    if (rc) return rc;
    const size_t need = unfused_ws_1d(B, Cin, Cout, modes);
    void* ws = user_ws;
    if (use_user_ws) {
        if (user_ws_bytes < need || !user_ws) return FNO_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(user_ws) & 255u) return FNO_ERR_ALIGN;
    }
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    if (!use_user_ws) {
        rc = internal_workspace(lease, st, need, &ws, stream);
        if (rc) return rc;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    rec_begin();
    return rec_end(hs, run_unfused_1d(B, Cin, Cout, N, modes, x, static_cast<const float2*>(w), out, ws,
                                      st->twiddle, hs, epi));
}

// ---------------------------------------------------------------------------
// backward pass
// ---------------------------------------------------------------------------

// Outputs of a backward call must not overlap any input or each other.
int check_backward(const float* x, const void* w, const float* g, const float* gx, const void* gw, size_t xbytes,
                   size_t wbytes, size_t gbytes) {
    if (!x || !w || !g || (!gx && !gw)) return FNO_ERR_NULL;
    if (misaligned(x) || misaligned(w) || misaligned(g) || (gx && misaligned(gx)) || (gw && misaligned(gw)))
        return FNO_ERR_ALIGN;
    if (gx && (overlap(gx, xbytes, x, xbytes) || overlap(gx, xbytes, w, wbytes) || overlap(gx, xbytes, g, gbytes)))
        return FNO_ERR_ALIAS;
    if (gw && (overlap(gw, wbytes, x, xbytes) || overlap(gw, wbytes, w, wbytes) || overlap(gw, wbytes, g, gbytes) ||
               (gx && overlap(gw, wbytes, gx, xbytes))))
        return FNO_ERR_ALIAS;
    return FNO_OK;
}

// Workspace of the backward pass: [R (staged transforms only)] [X] [G] [Z]
// [W^H], the spectra in the layout of the forward schedule for the shape.
struct BackwardPlan {
    bool small;
    SpecLayout lx, lg;
    size_t r_bytes, x_bytes, g_bytes, z_bytes, wt_bytes, wg_bytes;
    size_t total() const { return r_bytes + x_bytes + g_bytes + z_bytes + wt_bytes + wg_bytes; }
};

BackwardPlan backward_plan_2d(const Shape2d& s) {
    BackwardPlan p;
    const int64_t m = (int64_t)2 * s.mx * s.my;
    p.small = small_path(s);
    p.lx = p.small ? tiled_layout(s.Cin, m) : canonical_layout(s.Cin, m);
    p.lg = p.small ? tiled_layout(s.Cout, m) : canonical_layout(s.Cout, m);
    p.r_bytes = p.small ? 0
                        : align_up((size_t)s.B * (size_t)(s.Cin > s.Cout ? s.Cin : s.Cout) * s.H * s.my *
                                   sizeof(float2));
    p.x_bytes = align_up((size_t)layout_elems(p.lx, s.B) * sizeof(float2));
    p.g_bytes = align_up((size_t)layout_elems(p.lg, s.B) * sizeof(float2));
    p.z_bytes = p.x_bytes;
    p.wt_bytes = align_up((size_t)m * s.Cin * s.Cout * sizeof(float2));
    p.wg_bytes = align_up(weight_grad_workspace(s.B, s.Cin, s.Cout, m));
    return p;
}

int run_backward_2d(const Shape2d& s, const float* x, const float2* w, const float* g, float* gx, float2* gw,
                    void* ws, const float2* tw, hipStream_t st) {
    const BackwardPlan p = backward_plan_2d(s);
    const int64_t m = (int64_t)2 * s.mx * s.my;
    char* q = static_cast<char*>(ws);
    float2* r = reinterpret_cast<float2*>(q);
    q += p.r_bytes;
    float2* xh = reinterpret_cast<float2*>(q);
    q += p.x_bytes;
    float2* gh = reinterpret_cast<float2*>(q);
    q += p.g_bytes;
    float2* zh = reinterpret_cast<float2*>(q);
    q += p.z_bytes;
    float2* wt = reinterpret_cast<float2*>(q);
    q += p.wt_bytes;
    void* wg_ws = q;
    auto forward = [&](int64_t C, const float* in, float2* out_h, const SpecLayout& lay) {
        return p.small ? run_forward2d_small(s, C, in, out_h, lay, tw, st)
                       : run_forward2d_staged(s, C, in, out_h, r, tw, st);
    };
    int rc = forward(s.Cout, g, gh, p.lg);
    if (rc) return rc;
    if (gw) {
        rc = forward(s.Cin, x, xh, p.lx);
        if (rc) return rc;
        rec_kernel("wgrad", st);
        int splits = 1;
        hipError_t e = launch_weight_grad(xh, p.lx, gh, p.lg, gw, s.B, s.Cin, s.Cout, m, s.my, nyquist(s.W), wg_ws,
                                          p.wg_bytes, &splits, st);
        if (e != hipSuccess) return hip_fail(e);
        if (splits > 1) {
            rec_kernel("wgrad_reduce", st);
            e = launch_weight_grad_reduce(wg_ws, gw, s.Cin, s.Cout, m, splits, s.my, nyquist(s.W), st);
            if (e != hipSuccess) return hip_fail(e);
        }
    }
    if (gx) {
        rc = run_mix_adjoint(gh, p.lg, w, wt, zh, p.lx, s.B, s.Cout, s.Cin, m, st);
        if (rc) return rc;
        rc = p.small ? run_inverse2d_small(s, s.Cin, zh, gx, p.lx, tw, st)
                     : run_inverse2d_staged(s, s.Cin, zh, gx, r, tw, st);
        if (rc) return rc;
    }
    return FNO_OK;
}

int backward2d_common(const float* x, const void* w, const float* g, float* gx, void* gw, int B, int Cin, int Cout,
                      int H, int W, int mx, int my, void* stream) {
    int rc = check_dims_2d(B, Cin, H, W, mx, my);
    if (rc) return rc;
    if (Cout < 1) return FNO_ERR_SHAPE;
    const size_t xbytes = (size_t)B * Cin * H * W * sizeof(float);
    const size_t gbytes = (size_t)B * Cout * H * W * sizeof(float);
    const size_t wbytes = (size_t)2 * mx * my * Cin * Cout * sizeof(float2);
    rc = check_backward(x, w, g, gx, gw, xbytes, wbytes, gbytes);
    if (rc) return rc;
    const Shape2d s = make2d(B, Cin, Cout, H, W, mx, my);
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    rc = internal_workspace(lease, st, backward_plan_2d(s).total(), &ws, stream);
    if (rc) return rc;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    rec_begin();
    return rec_end(hs, run_backward_2d(s, x, static_cast<const float2*>(w), g, gx, static_cast<float2*>(gw), ws,
                                       st->twiddle, hs));
}

int backward1d_common(const float* x, const void* w, const float* g, float* gx, void* gw, int B, int Cin, int Cout,
                      int N, int modes, void* stream) {
    int rc = check_dims_1d(B, Cin, N, modes);
    if (rc) return rc;
    if (Cout < 1) return FNO_ERR_SHAPE;
    const size_t xbytes = (size_t)B * Cin * N * sizeof(float);
    const size_t gbytes = (size_t)B * Cout * N * sizeof(float);
    const size_t wbytes = (size_t)modes * Cin * Cout * sizeof(float2);
    rc = check_backward(x, w, g, gx, gw, xbytes, wbytes, gbytes);
    if (rc) return rc;
    const size_t xb = align_up((size_t)B * Cin * modes * sizeof(float2));
    const size_t gb = align_up((size_t)B * Cout * modes * sizeof(float2));
    const size_t wtb = align_up((size_t)modes * Cin * Cout * sizeof(float2));
    const size_t wgb = align_up(weight_grad_workspace(B, Cin, Cout, modes));
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    void* ws = nullptr;
    rc = internal_workspace(lease, st, 2 * xb + gb + wtb + wgb, &ws, stream);
    if (rc) return rc;
    char* q = static_cast<char*>(ws);
    float2* xh = reinterpret_cast<float2*>(q);
    float2* zh = reinterpret_cast<float2*>(q + xb);
    float2* gh = reinterpret_cast<float2*>(q + 2 * xb);
    float2* wt = reinterpret_cast<float2*>(q + 2 * xb + gb);
    void* wg_ws = q + 2 * xb + gb + wtb;
    const SpecLayout lx = canonical_layout(Cin, modes), lg = canonical_layout(Cout, modes);
    const float scale = (float)(1.0 / std::sqrt((double)N));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const float2* wc = static_cast<const float2*>(w);
    auto run = [&]() -> int {
        rec_kernel("rows_fwd", hs);
        hipError_t e = rows_fwd_n(g, gh, (int64_t)B * Cout, N, modes, modes, scale, st->twiddle, hs);
        if (e != hipSuccess) return hip_fail(e);
        if (gw) {
            rec_kernel("rows_fwd", hs);
            e = rows_fwd_n(x, xh, (int64_t)B * Cin, N, modes, modes, scale, st->twiddle, hs);
            if (e != hipSuccess) return hip_fail(e);
            rec_kernel("wgrad", hs);
            int splits = 1;
            e = launch_weight_grad(xh, lx, gh, lg, static_cast<float2*>(gw), B, Cin, Cout, modes, modes, nyquist(N), wg_ws,
                                   wgb, &splits, hs);
            if (e != hipSuccess) return hip_fail(e);
            if (splits > 1) {
                rec_kernel("wgrad_reduce", hs);
                e = launch_weight_grad_reduce(wg_ws, static_cast<float2*>(gw), Cin, Cout, modes, splits, modes,
                                              nyquist(N), hs);
                if (e != hipSuccess) return hip_fail(e);
            }
        }
        if (gx) {
            const int mrc = run_mix_adjoint(gh, lg, wc, wt, zh, lx, B, Cout, Cin, modes, hs);
            if (mrc) return mrc;
            rec_kernel("rows_inv", hs);
            e = rows_inv_n(zh, gx, (int64_t)B * Cin, N, modes, modes, scale, st->twiddle, hs);
            if (e != hipSuccess) return hip_fail(e);
        }
        return FNO_OK;
    };
    rec_begin();
    return rec_end(hs, run());
}

}  // namespace

LaunchEvents take_launch_events() {
    const LaunchEvents e = g_pending;
    g_pending = LaunchEvents{};
    return e;
}
}  // namespace fno

using namespace fno;

extern "C" {

int fno_version(void) { return kVersion; }

const char* fno_status_string(int status) {
    switch (status) {
        case FNO_OK: return "ok";
        case FNO_ERR_NULL: return "a required pointer is NULL";
        case FNO_ERR_SHAPE: return "a size is out of range or has a prime factor above 7";
        case FNO_ERR_MODES: return "mode counts out of range (need 1<=mx, 2*mx<=H, 1<=my<=W/2+1)";
        case FNO_ERR_ALIAS: return "output overlaps an input";
        case FNO_ERR_ALIGN: return "a pointer is not suitably aligned";
        case FNO_ERR_NOMEM: return "device workspace allocation failed";
        case FNO_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        case FNO_ERR_WORKSPACE: return "caller workspace missing or too small";
        case FNO_ERR_CAPTURE: return "a table or workspace would have to be allocated while the stream is captured";
        case FNO_ERR_TOO_LARGE: return "the shape needs more scratch than the fixed device array of the no-allocation call holds";
        case FNO_ERR_NOT_INIT: return "fno_init has not been called on this device";
        default: return "unknown status";
    }
}

int fno_last_hip_error(void) { return g_last_hip_error; }

int fno_init(void) {
    DeviceState* st = nullptr;
    int rc = device_state(&st, nullptr);
    if (rc) return rc;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!st->scratch) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
        st->scratch = p;
    }
    return FNO_OK;
}

int fno_set_timing_events(void** events, int n_events) {
    g_rec.events = (events && n_events > 0) ? events : nullptr;
    g_rec.n_events = g_rec.events ? n_events : 0;
    return FNO_OK;
}

int fno_last_kernel_count(void) { return g_rec.last_count; }

const char* fno_last_kernel_name(int k) {
    return (k >= 0 && k < g_rec.last_count) ? g_rec.last_names[k] : "";
}

int fno_spectral_conv2d(const float* x, const void* w, float* out, int B, int Cin, int Cout, int H, int W, int mx,
                        int my, void* stream) {
    return conv2d_common(x, w, out, B, Cin, Cout, H, W, mx, my, nullptr, 0, false, false, stream);
}

int fno_spectral_conv2d_unfused(const float* x, const void* w, float* out, int B, int Cin, int Cout, int H, int W,
                                int mx, int my, void* stream) {
    return conv2d_common(x, w, out, B, Cin, Cout, H, W, mx, my, nullptr, 0, false, true, stream);
}

int fno_spectral_conv2d_ws(const float* x, const void* w, float* out, int B, int Cin, int Cout, int H, int W,
                           int mx, int my, void* workspace, size_t ws_bytes, void* stream) {
    return conv2d_common(x, w, out, B, Cin, Cout, H, W, mx, my, workspace, ws_bytes, true, false, stream);
}

int fno_spectral_conv2d_noalloc(const float* x, const void* w, float* out, int B, int Cin, int Cout, int H, int W,
                                int mx, int my, void* stream) {
    int rc = check_dims_2d(B, Cin, H, W, mx, my);
    if (rc) return rc;
    if (Cout < 1) return FNO_ERR_SHAPE;
    // lengths other than powers of two would need their twiddle tables built
    if (!is_pow2(H) || !is_pow2(W)) return FNO_ERR_SHAPE;
    DeviceState* st = initialised_state();
    if (!st) return FNO_ERR_NOT_INIT;
    const size_t need = best_ws_2d(make2d(B, Cin, Cout, H, W, mx, my));
    if (need > kScratchBytes) return FNO_ERR_TOO_LARGE;
    // the device state exists, so conv2d_common's lookup allocates nothing
    return conv2d_common(x, w, out, B, Cin, Cout, H, W, mx, my, st->scratch, kScratchBytes, true, false, stream);
}

size_t fno_noalloc_scratch_bytes(void) { return kScratchBytes; }

int fno_spectral_conv1d(const float* x, const void* w, float* out, int B, int Cin, int Cout, int N, int modes,
                        void* stream) {
    return conv1d_common(x, w, out, B, Cin, Cout, N, modes, nullptr, 0, false, false, stream);
}

int fno_spectral_conv1d_unfused(const float* x, const void* w, float* out, int B, int Cin, int Cout, int N,
                                int modes, void* stream) {
    return conv1d_common(x, w, out, B, Cin, Cout, N, modes, nullptr, 0, false, true, stream);
}

int fno_spectral_conv1d_ws(const float* x, const void* w, float* out, int B, int Cin, int Cout, int N, int modes,
                           void* workspace, size_t ws_bytes, void* stream) {
    return conv1d_common(x, w, out, B, Cin, Cout, N, modes, workspace, ws_bytes, true, false, stream);
}

int fno_spectral_conv2d_gelu(const float* x, const void* w, const float* bias, const float* branch, float* out,
                             int B, int Cin, int Cout, int H, int W, int mx, int my, int branch_after,
                             void* stream) {
    int rc = check_dims_2d(B, Cin, H, W, mx, my);
    if (rc) return rc;
    if (Cout < 1) return FNO_ERR_SHAPE;
    if ((uint64_t)B * Cout * H > UINT32_MAX) return FNO_ERR_SHAPE;     // output rows indexed in 32 bits
    if (!out) return FNO_ERR_NULL;
    Epilogue epi;
    rc = check_epilogue(bias, branch, out, Cout, (size_t)B * Cout * H * W * sizeof(float), branch_after, &epi);
    if (rc) return rc;
    return conv2d_common(x, w, out, B, Cin, Cout, H, W, mx, my, nullptr, 0, false, false, stream, epi);
}

int fno_spectral_conv1d_gelu(const float* x, const void* w, const float* bias, const float* branch, float* out,
                             int B, int Cin, int Cout, int N, int modes, int branch_after, void* stream) {
    int rc = check_dims_1d(B, Cin, N, modes);
    if (rc) return rc;
    if (Cout < 1) return FNO_ERR_SHAPE;
    if ((uint64_t)B * Cout > UINT32_MAX) return FNO_ERR_SHAPE;         // output rows indexed in 32 bits
    if (!out) return FNO_ERR_NULL;
    Epilogue epi;
    rc = check_epilogue(bias, branch, out, Cout, (size_t)B * Cout * N * sizeof(float), branch_after, &epi);
    if (rc) return rc;
    return conv1d_common(x, w, out, B, Cin, Cout, N, modes, nullptr, 0, false, false, stream, epi);
}

int fno_spectral_filter2d(const float* x, const void* mask, float* out, int B, int C, int H, int W, int mx, int my,
                          void* stream) {
    return filter2d_common(x, mask, out, B, C, H, W, mx, my, stream);
}

int fno_spectral_filter1d(const float* x, const void* mask, float* out, int B, int C, int N, int modes,
                          void* stream) {
    return filter1d_common(x, mask, out, B, C, N, modes, stream);
}

int fno_linear_conv_length(int n, int k) { return linconv_len(n, k); }

int fno_linear_conv2d_prepare(const float* k, void* wspec, int Cin, int Cout, int H, int W, int kh, int kw,
                              void* stream) {
    return linconv2d_prepare(k, wspec, Cin, Cout, H, W, kh, kw, stream);
}

int fno_linear_conv2d(const float* x, const void* wspec, float* out, int B, int Cin, int Cout, int H, int W, int kh,
                      int kw, int crop_h, int crop_w, int Ho, int Wo, void* stream) {
    return linconv2d_run(x, wspec, out, B, Cin, Cout, H, W, kh, kw, crop_h, crop_w, Ho, Wo, stream);
}

int fno_linear_conv1d_prepare(const float* k, void* wspec, int Cin, int Cout, int N, int K, void* stream) {
    return linconv1d_prepare(k, wspec, Cin, Cout, N, K, stream);
}

int fno_linear_conv1d(const float* x, const void* wspec, float* out, int B, int Cin, int Cout, int N, int K,
                      int crop, int No, void* stream) {
    return linconv1d_run(x, wspec, out, B, Cin, Cout, N, K, crop, No, stream);
}

size_t fno_workspace_size_2d(int B, int Cin, int Cout, int H, int W, int mx, int my) {
    if (check_dims_2d(B, Cin, H, W, mx, my) || Cout < 1) return 0;
    return best_ws_2d(make2d(B, Cin, Cout, H, W, mx, my));
}

size_t fno_workspace_size_1d(int B, int Cin, int Cout, int N, int modes) {
    if (check_dims_1d(B, Cin, N, modes) || Cout < 1) return 0;
    return unfused_ws_1d(B, Cin, Cout, modes);
}

int fno_forward2d(const float* x, void* xh, int B, int C, int H, int W, int mx, int my, void* stream) {
    int rc = check_dims_2d(B, C, H, W, mx, my);
    if (rc) return rc;
    if (!x || !xh) return FNO_ERR_NULL;
    if (misaligned(x) || misaligned(xh)) return FNO_ERR_ALIGN;
    const size_t xbytes = (size_t)B * C * H * W * sizeof(float);
    const size_t hbytes = (size_t)B * C * 2 * mx * my * sizeof(float2);
    if (overlap(x, xbytes, xh, hbytes)) return FNO_ERR_ALIAS;
    const Shape2d s = make2d(B, C, C, H, W, mx, my);
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    float2* out = static_cast<float2*>(xh);
    if (small_path(s)) {
        rec_begin();
        return rec_end(hs, run_forward2d_small(s, C, x, out, canonical_layout(C, 2 * mx * my), st->twiddle, hs));
    }
    void* ws = nullptr;
    rc = internal_workspace(lease, st, (size_t)B * C * H * my * sizeof(float2), &ws, stream);
    if (rc) return rc;
    rec_begin();
    return rec_end(hs, run_forward2d_staged(s, C, x, out, static_cast<float2*>(ws), st->twiddle, hs));
}

int fno_inverse2d(const void* yh, float* out, int B, int C, int H, int W, int mx, int my, void* stream) {
    int rc = check_dims_2d(B, C, H, W, mx, my);
    if (rc) return rc;
    if (!yh || !out) return FNO_ERR_NULL;
    if (misaligned(yh) || misaligned(out)) return FNO_ERR_ALIGN;
    const size_t obytes = (size_t)B * C * H * W * sizeof(float);
    const size_t hbytes = (size_t)B * C * 2 * mx * my * sizeof(float2);
    if (overlap(out, obytes, yh, hbytes)) return FNO_ERR_ALIAS;
    const Shape2d s = make2d(B, C, C, H, W, mx, my);
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const float2* in = static_cast<const float2*>(yh);
    if (small_path(s)) {
        rec_begin();
        return rec_end(hs, run_inverse2d_small(s, C, in, out, canonical_layout(C, 2 * mx * my), st->twiddle, hs));
    }
    void* ws = nullptr;
    rc = internal_workspace(lease, st, (size_t)B * C * H * my * sizeof(float2), &ws, stream);
    if (rc) return rc;
    rec_begin();
    return rec_end(hs, run_inverse2d_staged(s, C, in, out, static_cast<float2*>(ws), st->twiddle, hs));
}

int fno_mix(const void* xh, const void* w, void* yh, int B, int Cin, int Cout, int M, void* stream) {
    if (B < 1 || Cin < 1 || Cout < 1 || M < 1) return FNO_ERR_SHAPE;
    if (!xh || !w || !yh) return FNO_ERR_NULL;
    if (misaligned(xh) || misaligned(w) || misaligned(yh)) return FNO_ERR_ALIGN;
    const size_t ybytes = (size_t)B * Cout * M * sizeof(float2);
    if (overlap(xh, (size_t)B * Cin * M * sizeof(float2), yh, ybytes) ||
        overlap(w, (size_t)M * Cin * Cout * sizeof(float2), yh, ybytes))
        return FNO_ERR_ALIAS;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    rec_begin();
    return rec_end(hs, run_mix(static_cast<const float2*>(xh), canonical_layout(Cin, M), static_cast<const float2*>(w),
                               static_cast<float2*>(yh), canonical_layout(Cout, M), B, Cin, Cout, M, hs));
}

int fno_forward1d(const float* x, void* xh, int B, int C, int N, int modes, void* stream) {
    int rc = check_dims_1d(B, C, N, modes);
    if (rc) return rc;
    if (!x || !xh) return FNO_ERR_NULL;
    if (misaligned(x) || misaligned(xh)) return FNO_ERR_ALIGN;
    if (overlap(x, (size_t)B * C * N * sizeof(float), xh, (size_t)B * C * modes * sizeof(float2)))
        return FNO_ERR_ALIAS;
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    const float scale = (float)(1.0 / std::sqrt((double)N));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    rec_begin();
    rec_kernel("rows_fwd", hs);
    hipError_t e = rows_fwd_n(x, static_cast<float2*>(xh), (int64_t)B * C, N, modes, modes, scale,
                                   st->twiddle, hs);
    return rec_end(hs, e == hipSuccess ? FNO_OK : hip_fail(e));
}

int fno_spectral_conv2d_backward(const float* x, const void* w, const float* grad_out, float* grad_x, void* grad_w,
                                 int B, int Cin, int Cout, int H, int W, int mx, int my, void* stream) {
    return backward2d_common(x, w, grad_out, grad_x, grad_w, B, Cin, Cout, H, W, mx, my, stream);
}

int fno_spectral_conv1d_backward(const float* x, const void* w, const float* grad_out, float* grad_x, void* grad_w,
                                 int B, int Cin, int Cout, int N, int modes, void* stream) {
    return backward1d_common(x, w, grad_out, grad_x, grad_w, B, Cin, Cout, N, modes, stream);
}

int fno_inverse1d(const void* yh, float* out, int B, int C, int N, int modes, void* stream) {
    int rc = check_dims_1d(B, C, N, modes);
    if (rc) return rc;
    if (!yh || !out) return FNO_ERR_NULL;
    if (misaligned(yh) || misaligned(out)) return FNO_ERR_ALIGN;
    if (overlap(out, (size_t)B * C * N * sizeof(float), yh, (size_t)B * C * modes * sizeof(float2)))
        return FNO_ERR_ALIAS;
    DeviceState* st = nullptr;
    WsLease lease;
    rc = device_state(&st, stream);
    if (rc) return rc;
    const float scale = (float)(1.0 / std::sqrt((double)N));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    rec_begin();
    rec_kernel("rows_inv", hs);
    hipError_t e = rows_inv_n(static_cast<const float2*>(yh), out, (int64_t)B * C, N, modes, modes,
                                   scale, st->twiddle, hs);
    return rec_end(hs, e == hipSuccess ? FNO_OK : hip_fail(e));
}

}  // extern "C"
