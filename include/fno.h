/*
 * libfno -- Fourier-neural-operator spectral convolution on MI355X (gfx950).
 *
 * C ABI.  Every pointer argument named x, w, out, xh, yh, grad_out, grad_x,
 * grad_w, bias, branch, mask, k, wspec or workspace is DEVICE memory on the current HIP
 * device, owned by the caller; the library never frees caller memory.  `stream` is a hipStream_t passed as void*
 * (NULL = the null stream).  All calls only enqueue work on `stream` and
 * return without synchronising; a kernel fault shows up at the caller's next
 * synchronisation.
 *
 * Argument checks run on the host before anything is enqueued: when a check
 * fails the call returns a negative status and nothing runs.
 *
 * The operation (sources: the TurboFNO blog "FFT-GEMM-iFFT full-chain fused
 * GPU operator", sections 1, 2.2, 3.1, 3.3 and 4.4; the "FFT for operator
 * optimisation" blog, sections 1.2, 2.1 and 2.2):
 *
 *   forward, ortho:  X[b,i,kx,ky] = (HW)^-1/2 sum_{h,w} x[b,i,h,w] e^{-2 pi i (kx h/H + ky w/W)}
 *                    for ky in [0, W/2] (real-to-complex half spectrum)
 *   truncate:        kx in [0,mx) u [H-mx,H) and ky in [0,my).  Weight block 0
 *                    holds kx = r, block 1 holds kx = H-mx+r, r < mx.
 *   mix:             Y[b,o,s,r,ky] = sum_i X[b,i,s,r,ky] * w[s,r,ky,i,o]
 *                    (plain complex product, no conjugate)
 *   inverse, ortho:  zero-fill every other mode, complex inverse along H,
 *                    complex-to-real inverse along W (the imaginary parts of
 *                    the ky = 0 and ky = W/2 bins do not contribute), scaled
 *                    by (HW)^-1/2.
 *
 * Layouts (row-major, contiguous, last index fastest):
 *   x    float32   [B][Cin][H][W]         (1D: [B][Cin][N])
 *   w    complex64 [2][mx][my][Cin][Cout] (1D: [modes][Cin][Cout])
 *   out  float32   [B][Cout][H][W]        (1D: [B][Cout][N])
 *   complex64 = interleaved (re, im) float32 pairs, as torch.complex64.
 *
 * Limits: 1 <= B, Cin, Cout; H and W 7-smooth (2^a 3^b 5^c 7^d) with
 * 2 <= H, W <= 4096 (1D: the same for N); 1 <= mx, 2*mx <= H;
 * 1 <= my <= W/2+1 (floor).  Powers of two take the specialised kernels;
 * other lengths take mixed-radix (4, 2, 3, 5, 7) stage kernels (the FFT
 * blog, section 6.2, on non-power-of-two sizes); the first call with a new
 * such length on a device builds that length's twiddle table (a device
 * allocation and a synchronous copy, like the first use of a workspace).
 * (1D: 1 <= modes <= N/2+1).  x, w, out must be 16-byte aligned and x must
 * not overlap out.  `out` is fully overwritten.
 */
#ifndef LIBFNO_FNO_H
#define LIBFNO_FNO_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fno_status {
    FNO_OK = 0,
    FNO_ERR_NULL = -1,       /* a required pointer is NULL */
    FNO_ERR_SHAPE = -2,      /* a size is out of range or has a prime factor above 7 */
    FNO_ERR_MODES = -3,      /* mx / my / modes out of range */
    FNO_ERR_ALIAS = -4,      /* x and out overlap */
    FNO_ERR_ALIGN = -5,      /* a pointer is not 16-byte aligned */
    FNO_ERR_NOMEM = -6,      /* the internal workspace could not be allocated */
    FNO_ERR_HIP = -7,        /* a HIP runtime call or kernel launch failed */
    FNO_ERR_WORKSPACE = -8,  /* caller workspace missing or smaller than required */
    FNO_ERR_CAPTURE = -9,    /* a table or workspace would have to be allocated while
                                the stream is being captured into a graph */
    FNO_ERR_TOO_LARGE = -10, /* shape needs more than fno_spectral_conv2d_noalloc's fixed scratch */
    FNO_ERR_NOT_INIT = -11   /* fno_init has not been called on the current device */
};

/* Library version as major*10000 + minor*100 + patch. */
int fno_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char* fno_status_string(int status);

/* The hipError_t of the last FNO_ERR_HIP on the calling thread (0 if none). */
int fno_last_hip_error(void);

/*
 * Builds the calling thread's current device's state: the twiddle table of
 * the power-of-two transforms (a device allocation and a synchronous copy).
 * Any other call does this on its first use of a device; calling it first
 * lets a caller capture a later call into a graph without an eager call
 * before (the stream's internal workspace still needs one eager call, or use
 * the _ws variants).  Idempotent; FNO_OK or FNO_ERR_NOMEM / FNO_ERR_HIP.
 */
int fno_init(void);

/*
 * 2D spectral convolution (TurboFNO blog, sections 1 and 2.2; FFT blog
 * sections 2.1-2.2).  Picks the fastest implemented schedule for the shape:
 * grids of at most 1024 points with at most 8 channels in and out run as one
 * kernel, one workgroup per batch item with its truncated spectra on chip
 * (no workspace); other grids up to 128 per side as three kernels (forward,
 * channel mix, inverse, the spectra in workspace); longer rows and taller
 * grids as five (rows, columns, mix, columns, rows).
 * Uses an internal workspace per (device, stream), following the FFT blog's
 * plan and work-area reuse (sections 2.2 and 5.3): grow-only, allocated on
 * first use and kept until process exit, so calls on different streams may
 * overlap in time.  Growing it waits for the work already enqueued on that
 * stream, then frees the old buffer; host threads calling on the same stream
 * are serialised from workspace lookup until their kernels are enqueued.
 * The _ws variants take caller-owned scratch instead.
 *
 * HIP graph capture: every call enqueues kernels only (no memset or copy
 * nodes).  A call that would have to allocate while its stream is being
 * captured (the device's twiddle table before fno_init or any eager call; a
 * new or larger internal workspace; the table of a new non-power-of-two
 * length) returns FNO_ERR_CAPTURE and enqueues nothing.  A captured graph
 * holds the workspace's address: a later call on the same stream that needs
 * a larger workspace reallocates it, after which graphs captured on that
 * stream must not be replayed.
 */
int fno_spectral_conv2d(const float* x, const void* w, float* out,
                        int B, int Cin, int Cout, int H, int W, int mx, int my,
                        void* stream);

/*
 * 1D spectral convolution along a sequence of length N (FFT blog, section 3.2:
 * FFT token mixing; the weight has one block because a length-N axis has no
 * second frequency axis to truncate).  Scale N^-1/2 on each transform.
 */
int fno_spectral_conv1d(const float* x, const void* w, float* out,
                        int B, int Cin, int Cout, int N, int modes, void* stream);

/*
 * Unfused schedules of the same hand-written stages, kept for ablation
 * (TurboFNO blog, sections 1 and 2.1: FFT, GEMM and iFFT as separate passes
 * with the spectra round-tripping through device memory): row transforms,
 * column transforms, mix, column inverse, row inverse as five kernels, the
 * row spectra in device memory.  Same arguments and results as the calls
 * above.  The 1D call has no separate fused schedule: fno_spectral_conv1d_unfused
 * runs the same three kernels as fno_spectral_conv1d.
 */
int fno_spectral_conv2d_unfused(const float* x, const void* w, float* out,
                                int B, int Cin, int Cout, int H, int W, int mx, int my,
                                void* stream);
int fno_spectral_conv1d_unfused(const float* x, const void* w, float* out,
                                int B, int Cin, int Cout, int N, int modes, void* stream);

/*
 * Bytes of caller workspace the _ws calls need for this shape (0 when the
 * fastest schedule needs none): the query half of the FFT blog's plan /
 * work-area pattern (sections 2.2 and 5.3).  Never fails; returns 0 for
 * invalid shapes.
 */
size_t fno_workspace_size_2d(int B, int Cin, int Cout, int H, int W, int mx, int my);
size_t fno_workspace_size_1d(int B, int Cin, int Cout, int N, int modes);

/*
 * As fno_spectral_conv2d / _1d, but all scratch lives in `workspace`
 * (device memory, at least fno_workspace_size_* bytes, 256-byte aligned,
 * caller-owned; the FFT blog's caller-provided work area, sections 2.2 and
 * 5.3).  Returns FNO_ERR_WORKSPACE if it is too small or NULL while a
 * non-zero size is needed.  These calls allocate nothing once the device's
 * twiddle table exists (fno_init or any earlier call on the device) and, for
 * a length that is not a power of two, once that length's table exists (any
 * earlier call with that length); otherwise they build those tables first,
 * or return FNO_ERR_CAPTURE while the stream is being captured.
 */
int fno_spectral_conv2d_ws(const float* x, const void* w, float* out,
                           int B, int Cin, int Cout, int H, int W, int mx, int my,
                           void* workspace, size_t ws_bytes, void* stream);
int fno_spectral_conv1d_ws(const float* x, const void* w, float* out,
                           int B, int Cin, int Cout, int N, int modes,
                           void* workspace, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): fno_spectral_conv2d
 * with its scratch (the truncated spectra) in a fixed device array of
 * fno_noalloc_scratch_bytes() bytes (64 MiB), which every device that loads
 * the library holds until the process ends.  The call allocates and frees
 * nothing.  Before the first call on a device, call fno_init on it (it looks
 * up that device's address of the array and builds the twiddle table);
 * otherwise FNO_ERR_NOT_INIT.  H and W must be powers of two (other lengths
 * would need a table built; FNO_ERR_SHAPE); a shape whose spectra need more
 * than the array holds returns FNO_ERR_TOO_LARGE (the 128x128 workload with
 * B=32, Cin=Cout=64 and 32x32 modes needs exactly 64 MiB).  Nothing in the
 * array needs to start at zero: every call writes the spectra it reads.  All
 * calls on one device share the one array, which keeps the last call's
 * contents: calls that overlap in time on one device (other streams or host
 * threads) race on it and must be serialised by the caller.  Same arguments,
 * results and other errors as fno_spectral_conv2d.
 */
int fno_spectral_conv2d_noalloc(const float* x, const void* w, float* out,
                                int B, int Cin, int Cout, int H, int W, int mx, int my,
                                void* stream);
size_t fno_noalloc_scratch_bytes(void);

/*
 * Stage calls, for stage-by-stage comparison of the intermediate spectra
 * (FFT blog, section 6.4).  The truncated spectra use the weight's mode
 * order: xh complex64 [B][C][2][mx][my] (1D: [B][C][modes]).
 *
 *   fno_forward2d:  x[B][C][H][W] -> xh, ortho scale included.
 *   fno_mix:        xh[B][Cin][M], w[M][Cin][Cout] -> yh[B][Cout][M], M modes.
 *   fno_inverse2d:  yh[B][C][2][mx][my] -> out[B][C][H][W], ortho scale included.
 *   fno_forward1d / fno_inverse1d: the same for sequences.
 * fno_forward2d / fno_inverse2d use the internal workspace (see above).
 */
int fno_forward2d(const float* x, void* xh, int B, int C, int H, int W, int mx, int my,
                  void* stream);
int fno_mix(const void* xh, const void* w, void* yh, int B, int Cin, int Cout, int M,
            void* stream);
int fno_inverse2d(const void* yh, float* out, int B, int C, int H, int W, int mx, int my,
                  void* stream);
int fno_forward1d(const float* x, void* xh, int B, int C, int N, int modes, void* stream);
int fno_inverse1d(const void* yh, float* out, int B, int C, int N, int modes, void* stream);

/*
 * Backward pass: gradients of a real loss L through fno_spectral_conv2d /
 * _1d, given grad_out = dL/dout (float32, the layout of out):
 *
 *   grad_x  float32   [B][Cin][H][W]           dL/dx
 *           = the forward chain applied to grad_out with the conjugate-
 *             transposed weight w^H[s,r,ky,o,i] = conj w[s,r,ky,i,o]
 *   grad_w  complex64 [2][mx][my][Cin][Cout]   dL/dRe(w) + i dL/dIm(w)
 *           = c_ky sum_b conj(X[b,i,s,r,ky]) G[b,o,s,r,ky]
 *
 * X and G are the truncated forward transforms of x and grad_out, c_ky the
 * complex-to-real weight (1 for ky = 0 and ky = W/2, 2 otherwise) (chain
 * rule through the TurboFNO blog's section 2.2 product and the FFT blog's
 * section 2.2 C2R).  1D: the same with one weight block [modes][Cin][Cout].
 * x, w and grad_out are required; grad_x or grad_w may be NULL to skip that
 * gradient, not both.  Outputs are fully overwritten and must not overlap
 * any input or each other.  Uses the internal workspace (see
 * fno_spectral_conv2d).
 */
int fno_spectral_conv2d_backward(const float* x, const void* w, const float* grad_out,
                                 float* grad_x, void* grad_w,
                                 int B, int Cin, int Cout, int H, int W, int mx, int my,
                                 void* stream);
int fno_spectral_conv1d_backward(const float* x, const void* w, const float* grad_out,
                                 float* grad_x, void* grad_w,
                                 int B, int Cin, int Cout, int N, int modes, void* stream);

/*
 * Spectral convolution with the fused layer tail (the FFT blog's fused
 * operator, sections 5.1-5.2: the C2R output is activated with GELU and
 * added to a second, time-domain branch inside the kernel that writes the
 * output, section 6.2).  With conv = fno_spectral_conv2d(x, w):
 *
 *   branch_after = 0:  out = gelu(conv + bias[o] + branch)   (FNO-layer form)
 *   branch_after = 1:  out = gelu(conv + bias[o]) + branch   (the blog's order)
 *
 * gelu(u) = u (1 + erf(u / sqrt 2)) / 2.  bias float32 [Cout] (4-byte
 * aligned) and branch float32 (the shape and layout of out, 16-byte aligned)
 * are optional: NULL reads as zero.  Neither may overlap out (FNO_ERR_ALIAS);
 * branch_after outside {0, 1} is FNO_ERR_SHAPE.  Everything else as
 * fno_spectral_conv2d / fno_spectral_conv1d (internal workspace).
 */
int fno_spectral_conv2d_gelu(const float* x, const void* w, const float* bias,
                             const float* branch, float* out,
                             int B, int Cin, int Cout, int H, int W, int mx, int my,
                             int branch_after, void* stream);
int fno_spectral_conv1d_gelu(const float* x, const void* w, const float* bias,
                             const float* branch, float* out,
                             int B, int Cin, int Cout, int N, int modes,
                             int branch_after, void* stream);

/*
 * Diagonal global filter (the learnable frequency mask of the TurboFNO blog,
 * section 5.2: fft2 -> mask -> ifft2; the frequency-domain token mixing of
 * the FFT blog, section 3.2: R2C along the sequence -> learnable complex
 * mask -> C2R): the spectral convolution with the channel mix replaced by
 * one complex weight per kept mode and channel,
 *
 *   Y[b,c,s,r,ky] = X[b,c,s,r,ky] * mask[s,r,ky,c]      (1D: mask[ky,c])
 *
 * then zero-fill and the ortho C2R inverse, exactly as fno_spectral_conv2d.
 * x float32 [B][C][H][W] (1D: [B][C][N]), mask complex64 [2][mx][my][C]
 * (1D: [modes][C]), out float32 of x's shape.  Keeping every mode (mx = H/2,
 * my = W/2 + 1) gives the untruncated global filter.  Checks and workspace
 * as fno_spectral_conv2d (out must not overlap x or mask).
 */
int fno_spectral_filter2d(const float* x, const void* mask, float* out,
                          int B, int C, int H, int W, int mx, int my, void* stream);
int fno_spectral_filter1d(const float* x, const void* mask, float* out,
                          int B, int C, int N, int modes, void* stream);

/*
 * Zero-padded linear convolution (the FFT blog, sections 2.1 and 5.1-5.2:
 * pad input and kernel, R2C, pointwise product, C2R, crop):
 *
 *   y[b,o,p,q] = sum_i sum_{dh<kh, dw<kw} x[b,i,p-dh,q-dw] k[o,i,dh,dw]
 *
 * (x zero outside its H x W grid; y is (H+kh-1) x (W+kw-1)), and
 * out[b,o,h,w] = y[b,o,h+crop_h,w+crop_w] for h < Ho, w < Wo ("same" output:
 * crop (kh-1)/2, (kw-1)/2 and Ho = H, Wo = W).  H, W may be any size.  Both
 * operands are zero-padded to PH x PW with PH = fno_linear_conv_length(H, kh),
 * PW = fno_linear_conv_length(W, kw) (the smallest even 7-smooth length
 * 2^a 3^b 5^c 7^d holding the full convolution: at most 8192, and not a
 * power of two above 4096; 0 when out of range; the 2D column length PH at
 * most 4096, else FNO_ERR_SHAPE), where the circular convolution equals the
 * linear one, and the
 * spectral convolution runs at full modes (mx = PH/2, my = PW/2+1) with the
 * weight spectrum
 *
 *   wspec[s][r][ky][i][o] = sqrt(PH PW) * (ortho R2C of the padded k[o][i])
 *
 * which fno_linear_conv2d_prepare computes from k float32 [Cout][Cin][kh][kw]
 * into wspec complex64 [2][PH/2][PW/2+1][Cin][Cout] (compute it once per
 * kernel and reuse it).  fno_linear_conv2d: x float32 [B][Cin][H][W], out
 * float32 [B][Cout][Ho][Wo]; the crop window must lie inside y
 * (FNO_ERR_SHAPE).  1D: k [Cout][Cin][K], wspec [PN/2+1][Cin][Cout] with
 * PN = fno_linear_conv_length(N, K), x [B][Cin][N], out [B][Cout][No] from
 * y[crop].  Internal workspace; out must not overlap x or wspec, wspec not k.
 */
int fno_linear_conv_length(int n, int k);
int fno_linear_conv2d_prepare(const float* k, void* wspec, int Cin, int Cout, int H, int W,
                              int kh, int kw, void* stream);
int fno_linear_conv2d(const float* x, const void* wspec, float* out, int B, int Cin, int Cout,
                      int H, int W, int kh, int kw, int crop_h, int crop_w, int Ho, int Wo,
                      void* stream);
int fno_linear_conv1d_prepare(const float* k, void* wspec, int Cin, int Cout, int N, int K,
                              void* stream);
int fno_linear_conv1d(const float* x, const void* wspec, float* out, int B, int Cin, int Cout,
                      int N, int K, int crop, int No, void* stream);

/*
 * Per-kernel timing for benchmarks and profilers.  While `events` is non-NULL,
 * every convolution or stage call made on the calling thread launches its
 * k-th kernel with events[2k] and events[2k+1] (hipEvent_t, created by the
 * caller) as the launch's start and stop events, so they hold that kernel's
 * own start and end timestamps; no extra work is queued between kernels.
 * Kernels whose pair lies beyond n_events-1 launch without events.  Pass NULL
 * to stop.  Returns FNO_OK.  fno_last_kernel_count / fno_last_kernel_name
 * report, for the calling thread's last successful call, how many kernels it
 * launched and their names (static storage; "" for an index out of range).
 */
int fno_set_timing_events(void** events, int n_events);
int fno_last_kernel_count(void);
const char* fno_last_kernel_name(int k);

#ifdef __cplusplus
}
#endif

#endif /* LIBFNO_FNO_H */
