// Device-side building blocks of libfno: complex arithmetic, small in-register
// DFTs and a Stockham FFT over rows held in LDS.
//
// Conventions: complex64 values are float2 (x = re, y = im).  SIGN = -1 is the
// forward transform exp(-2 pi i n k / N), SIGN = +1 the unnormalised inverse
// (TurboFNO blog, sections 2.1-2.2: row and column 1D transforms make the 2D
// transform; FFT blog, section 2.2: R2C / C2R with the N/2+1 half spectrum).
//
// Twiddles W_N^m = exp(-2 pi i m / N) for the Stockham passes come from one
// table of length kNMax that the host fills once per device in double
// precision (angle 2 pi m / kNMax with exact integer m) and rounds to float.
// The small radix-2/4/8/16 butterflies use the exact constants cos(pi/4),
// cos(pi/8), sin(pi/8) written out to float precision.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

namespace fno {

constexpr int kLog2NMax = 12;            // longest transform: 4096 points
constexpr int kNMax = 1 << kLog2NMax;    // twiddle table length
constexpr int kLdsElems = 4096;          // complex elements per LDS ping-pong buffer

constexpr float kSqrtHalf = 0.70710678118654752440f;  // cos(pi/4)

// Compile-time cos / sin of 2 pi e / N for the register-resident transforms:
// argument reduction to [0, pi/4] by octant symmetries, then Taylor series in
// double (terms to x^29; |x| <= pi/4 so the remainder is far below double
// rounding), rounded once to float.
constexpr double kPi = 3.14159265358979323846264338327950288;

constexpr double taylor_cos(double x) {
    double term = 1.0, sum = 1.0;
    for (int k = 1; k <= 15; ++k) {
        term *= -x * x / ((2.0 * k - 1.0) * (2.0 * k));
        sum += term;
    }
    return sum;
}
constexpr double taylor_sin(double x) {
    double term = x, sum = x;
    for (int k = 1; k <= 15; ++k) {
        term *= -x * x / ((2.0 * k) * (2.0 * k + 1.0));
        sum += term;
    }
    return sum;
}
// cos(2 pi e / n) and sin(2 pi e / n) for integer e, n a multiple of 8
constexpr double exact_cos(int e, int n) {
    e = ((e % n) + n) % n;
    const int oct = n / 8;                    // e in octant e / oct
    const int o = e / oct;
    const int r = e % oct;
    const double a = 2.0 * kPi * r / n;       // in [0, pi/4)
    const double b = 2.0 * kPi * (oct - r) / n;
    switch (o) {
        case 0: return taylor_cos(a);
        case 1: return taylor_sin(b);
        case 2: return -taylor_sin(a);
        case 3: return -taylor_cos(b);
        case 4: return -taylor_cos(a);
        case 5: return -taylor_sin(b);
        case 6: return taylor_sin(a);
        default: return taylor_cos(b);
    }
}
constexpr double exact_sin(int e, int n) { return exact_cos(e - n / 4, n); }

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cscale(float2 a, float s) { return make_float2(a.x * s, a.y * s); }
__device__ __forceinline__ float2 conj2(float2 a) { return make_float2(a.x, -a.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    // (a+bi)(c+di) = (ac-bd) + (ad+bc)i   (TurboFNO blog, section 2.2)
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cfma(float2 acc, float2 a, float2 b) {
    acc.x = fmaf(a.x, b.x, acc.x);
    acc.x = fmaf(-a.y, b.y, acc.x);
    acc.y = fmaf(a.x, b.y, acc.y);
    acc.y = fmaf(a.y, b.x, acc.y);
    return acc;
}

// v * (SIGN * i)
template <int SIGN>
__device__ __forceinline__ float2 mul_i(float2 v) {
    return SIGN < 0 ? make_float2(v.y, -v.x) : make_float2(-v.y, v.x);
}

// v * exp(SIGN * 2 pi i * E / N), N a power of two >= 8.  E is a template
// argument so the constants are folded at compile time.
template <int SIGN, int N, int E>
__device__ __forceinline__ float2 wmul(float2 v) {
    constexpr int e = E & (N - 1);
    if constexpr (e == 0) {
        return v;
    } else if constexpr (4 * e == N) {
        return mul_i<SIGN>(v);
    } else if constexpr (2 * e == N) {
        return make_float2(-v.x, -v.y);
    } else if constexpr (4 * e == 3 * N) {
        return mul_i<-SIGN>(v);
    } else if constexpr (8 * e == N || 8 * e == 3 * N || 8 * e == 5 * N || 8 * e == 7 * N) {
        // |cos| = |sin| = cos(pi/4): two adds and two multiplies
        constexpr float sc = exact_cos(e, N) < 0 ? -1.0f : 1.0f;
        constexpr float ss = SIGN * exact_sin(e, N) < 0 ? -1.0f : 1.0f;
        return make_float2((v.x * sc - v.y * ss) * kSqrtHalf, (v.x * ss + v.y * sc) * kSqrtHalf);
    } else {
        constexpr float c = (float)exact_cos(e, N);
        constexpr float s = (float)(SIGN * exact_sin(e, N));
        return make_float2(v.x * c - v.y * s, v.x * s + v.y * c);
    }
}

// Calls f(std::integral_constant<int, I>) for I = B, ..., E-1 in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        [[clang::always_inline]] f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// acc + v * exp(SIGN * 2 pi i * E / N) on fused multiply-adds (E and N
// compile-time): four instructions for a general factor instead of the six
// of a separate product and sum.
template <int SIGN, int N, int E>
__device__ __forceinline__ float2 wfma(float2 acc, float2 v) {
    constexpr int e = E & (N - 1);
    if constexpr (e == 0) {
        return cadd(acc, v);
    } else if constexpr (4 * e == N) {
        return cadd(acc, mul_i<SIGN>(v));
    } else if constexpr (2 * e == N) {
        return csub(acc, v);
    } else if constexpr (4 * e == 3 * N) {
        return cadd(acc, mul_i<-SIGN>(v));
    } else {
        constexpr float c = (float)exact_cos(e, N);
        constexpr float s = (float)(SIGN * exact_sin(e, N));
        return make_float2(fmaf(v.x, c, fmaf(-v.y, s, acc.x)), fmaf(v.x, s, fmaf(v.y, c, acc.y)));
    }
}

// Radix-2 butterfly lo = a + T b, hi = a - T b, T = exp(SIGN * 2 pi i * E / N)
// (E and N compile-time).  A general factor T = c + i s is applied as
// c (1 + i s/c) when |s| <= |c|, else as s (c/s + i): the product with the
// bracket takes two fused multiply-adds and each output two more, six in
// all instead of the eight of a product followed by a sum and a difference.
template <int SIGN, int N, int E>
__device__ __forceinline__ void bfly(float2 a, float2 b, float2& lo, float2& hi) {
    constexpr int e = E & (N - 1);
    if constexpr (e == 0) {
        lo = cadd(a, b);
        hi = csub(a, b);
    } else if constexpr (4 * e == N || 4 * e == 3 * N) {
        const float2 t = mul_i<4 * e == N ? SIGN : -SIGN>(b);
        lo = cadd(a, t);
        hi = csub(a, t);
    } else if constexpr (2 * e == N) {
        lo = csub(a, b);
        hi = cadd(a, b);
    } else {
        constexpr double c = exact_cos(e, N);
        constexpr double s = SIGN * exact_sin(e, N);
        constexpr bool by_c = (c < 0 ? -c : c) >= (s < 0 ? -s : s);
        constexpr float f = (float)(by_c ? c : s);
        constexpr float t = (float)(by_c ? s / c : c / s);
        float2 u;
        if constexpr (by_c) u = make_float2(fmaf(-t, b.y, b.x), fmaf(t, b.x, b.y));   // (1 + i t) b
        else u = make_float2(fmaf(t, b.x, -b.y), fmaf(t, b.y, b.x));                   // (t + i) b
        lo = make_float2(fmaf(f, u.x, a.x), fmaf(f, u.y, a.y));
        hi = make_float2(fmaf(-f, u.x, a.x), fmaf(-f, u.y, a.y));
    }
}

// In-register DFT of size R <= 64, natural order in and out:
// v[k] <- sum_r v[r] exp(SIGN 2 pi i r k / R).  Radix-2 decimation in time.
template <int R, int SIGN>
__device__ __forceinline__ void dft(float2 (&v)[R]) {
    static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "radix must be a power of two <= 64");
    if constexpr (R >= 2) {
        constexpr int HALF = R / 2;
        float2 e[HALF], o[HALF];
        static_for<0, HALF>([&](auto i) {
            e[i] = v[2 * i];
            o[i] = v[2 * i + 1];
        });
        dft<HALF, SIGN>(e);
        dft<HALF, SIGN>(o);
        static_for<0, HALF>([&](auto k) { bfly<SIGN, R, k>(e[k], o[k], v[k], v[k + HALF]); });
    }
}

// Sum of a value over the four lanes of its quad (DPP quad_perm [1,0,3,2]
// then [2,3,0,1]); every lane of the quad gets the sum.  All four lanes must
// be active.
__device__ __forceinline__ float quad_sum1(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float2 quad_sum(float2 v) { return make_float2(quad_sum1(v.x), quad_sum1(v.y)); }

// Workgroup barrier that orders LDS accesses only: global loads issued before
// it stay in flight (a plain __syncthreads would wait for them too), which
// lets a kernel prefetch the next item's inputs across its LDS phases.
// The scheduling barriers keep the compiler from moving arithmetic of the
// next phase above it (which would keep two phases' registers live at once).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    __builtin_amdgcn_sched_barrier(0);
}

// Orders LDS accesses between the lanes of one wave (LDS operations of a wave
// complete in issue order; this only stops the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3: 32-bit
// data format, no swizzle, no stride).  The hardware range-checks every
// access: a load at a byte offset >= bytes returns zero and such a store is
// dropped, so an offset of kBufferSkip turns a store off without a branch.
constexpr uint32_t kBufferSkip = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef unsigned int u32x2_t __attribute__((__vector_size__(2 * sizeof(unsigned int))));
typedef unsigned int u32x4_t __attribute__((__vector_size__(4 * sizeof(unsigned int))));

__device__ __forceinline__ float4 buffer_load_f4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

__device__ __forceinline__ float buffer_load_f1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ float2 buffer_load_f2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
}

__device__ __forceinline__ void buffer_store_f4(float4 a, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    u32x4_t v;
    v[0] = __float_as_uint(a.x);
    v[1] = __float_as_uint(a.y);
    v[2] = __float_as_uint(a.z);
    v[3] = __float_as_uint(a.w);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, 0);
}

// Non-temporal stores for a call's final outputs (never read back within
// the call): they stream to memory instead of staying dirty in the
// last-level cache, where their write-back would compete with the next
// reads.  Buffer form: cache-policy bit 1 (nt).
__device__ __forceinline__ void buffer_store_f4_nt(float4 a, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    u32x4_t v;
    v[0] = __float_as_uint(a.x);
    v[1] = __float_as_uint(a.y);
    v[2] = __float_as_uint(a.z);
    v[3] = __float_as_uint(a.w);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, 2);
}

__device__ __forceinline__ void nt_store(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void nt_store2(float2* p, float2 v) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    const f2v t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<f2v*>(p));
}

__device__ __forceinline__ void buffer_store_f2(float2 a, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    u32x2_t v;
    v[0] = __float_as_uint(a.x);
    v[1] = __float_as_uint(a.y);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, (int)soff, 0);
}

// Logical work index -> image.  Indices L and L + 8 (same XCD under
// round-robin workgroup dispatch, same step of the persistent loop when the
// grid is a multiple of 16) get images 2j and 2j + 1.
__device__ __forceinline__ int64_t paired_image(int64_t L, int64_t nimg) {
    const int64_t g = L >> 4;
    if ((g + 1) * 16 > nimg) return L;
    const int r = (int)(L & 15);
    return g * 16 + 2 * (r & 7) + (r >> 3);
}

// Twiddle exp(SIGN 2 pi i m / kNMax) from the host-built table of exp(-2 pi i m / kNMax).
template <int SIGN>
__device__ __forceinline__ float2 table_twiddle(const float2* __restrict__ tw, int m) {
    float2 t = tw[m];
    if (SIGN > 0) t.y = -t.y;
    return t;
}

// One radix-R Stockham pass (decimation in time, autosort) of an N-point
// transform whose sub-transforms of length NS are already done.  Butterfly j
// reads src[j + r N/R], twiddles by W_{NS R}^{r (j mod NS)}, runs a radix-R
// DFT and writes dst[(j - j mod NS) R + j mod NS + r NS].
template <int N, int NS, int R, int SIGN>
__device__ __forceinline__ void stockham_pass(const float2* src, float2* dst, int j,
                                              const float2* __restrict__ tw) {
    constexpr int STRIDE = N / R;
    constexpr int TW_STEP = kNMax / (NS * R);
    float2 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = src[j + r * STRIDE];
    const int k = j & (NS - 1);
    if constexpr (NS > 1) {
#pragma unroll
        for (int r = 1; r < R; ++r) v[r] = cmul(v[r], table_twiddle<SIGN>(tw, r * k * TW_STEP));
    }
    dft<R, SIGN>(v);
    const int base = (j - k) * R + k;
#pragma unroll
    for (int r = 0; r < R; ++r) dst[base + r * NS] = v[r];
}

// Full N = 2^LOG2N point transform of `nrows` rows (row stride `ld`) held in
// LDS buffer `a`, ping-ponging through `b`.  All threads of the block must
// call it.  Returns the buffer that holds the result (natural order).
template <int LOG2N, int SIGN, int DONE = 0>
__device__ __forceinline__ float2* fft_rows_lds(float2* a, float2* b, int nrows, int ld,
                                                const float2* __restrict__ tw, int tid, int nthr) {
    if constexpr (DONE >= LOG2N) {
        return a;
    } else {
        constexpr int REM = LOG2N - DONE;
        constexpr int RB = REM >= 4 ? 4 : REM;
        constexpr int R = 1 << RB;
        constexpr int N = 1 << LOG2N;
        constexpr int NS = 1 << DONE;
        constexpr int J = N / R;
        const int total = nrows * J;
        for (int idx = tid; idx < total; idx += nthr) {
            const int row = idx / J;
            const int j = idx & (J - 1);
            stockham_pass<N, NS, R, SIGN>(a + row * ld, b + row * ld, j, tw);
        }
        __syncthreads();
        return fft_rows_lds<LOG2N, SIGN, DONE + RB>(b, a, nrows, ld, tw, tid, nthr);
    }
}

}  // namespace fno
