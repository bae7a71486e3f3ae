// Half-spectrum bins of a real sequence from its packed complex transform,
// and back (FFT blog, section 2.2: R2C and C2R on the N/2 + 1 half
// spectrum), for the register transforms of the row kernels.
#pragma once

#include "fno_device.hpp"

namespace fno {

// Twice bin K (K <= Q/2) of the DFT of a real length-Q sequence s, from its
// packed transform Z = DFT_{Q/2}(s[2m] + i s[2m+1]):
//   2 Y[K] = (Z[K] + conj Z[-K]) - i W_Q^K (Z[K] - conj Z[-K]).
// The factor 2 is taken out with the output scale.
template <int Q, int K>
__device__ __forceinline__ float2 real_bin2(const float2 (&z)[Q / 2]) {
    constexpr int NZ = Q / 2;
    const float2 zk = z[K % NZ];
    const float2 zm = z[(NZ - K % NZ) % NZ];
    const float2 e = make_float2(zk.x + zm.x, zk.y - zm.y);
    const float2 o = make_float2(zk.y + zm.y, zm.x - zk.x);
    return wfma<-1, Q, K>(e, o);
}

// Packed C2R bin K (K < Q/2) from a Hermitian half spectrum H[0..Q/2]:
//   s[2m] + i s[2m+1] = IDFT_{Q/2}(Zp)[m],
//   Zp[K] = (H[K] + conj H[Q/2-K]) + i W_Q^{-K} (H[K] - conj H[Q/2-K]).
template <int Q, int K>
__device__ __forceinline__ float2 packed_bin(const float2 (&H)[Q / 2 + 1]) {
    constexpr int NZ = Q / 2;
    const float2 hk = H[K], hm = H[NZ - K];
    const float2 a = make_float2(hk.x + hm.x, hk.y - hm.y);
    const float2 b = make_float2(hk.x - hm.x, hk.y + hm.y);
    // i W_Q^{-K} b = W_Q^{-K} (i b)
    return wfma<1, Q, K>(a, make_float2(-b.y, b.x));
}

}  // namespace fno
