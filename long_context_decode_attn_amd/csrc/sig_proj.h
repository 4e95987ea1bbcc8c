// sig_proj.h - one random projection of a 128-value row, the arithmetic of the
// T_map stage ("HashAttention: Semantic Sparsity for Faster Inference", slide
// "A 32-bit signature makes scoring cheap", Eq. (1): bit b of the code is
// ReLU(sign(x . R[:, b]))).  Shared by the encoder and the TOPK pass that
// encodes its queries at its head.
//
// The projection is a chain of fp64 fused multiply-adds over the values in
// order, from 0: a bf16 or fp32 value times an fp32 value is exact in fp64 and
// the fixed chain fixes the rounding of the sum, so the code is reproducible
// bit for bit, including the sign of a projection near zero.
#pragma once

#include "common.h"

namespace lcda {

// Eight values of a row as floats (bf16: one 16-byte load; fp32: two).
__device__ __forceinline__ void load8f(const uint16_t* p, float (&f)[8]) {
    const u32x4 v = ld16(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[2 * k] = bf16_lo(v[k]);
        f[2 * k + 1] = bf16_hi(v[k]);
    }
}

__device__ __forceinline__ void load8f(const float* p, float (&f)[8]) {
    const u32x4 a = ld16(p), b = ld16(p + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f[k] = __uint_as_float(a[k]);
        f[4 + k] = __uint_as_float(b[k]);
    }
}

// A whole row as floats (one round of loads).
template <typename T>
__device__ __forceinline__ void load_row(const T* row, float (&xf)[kD]) {
#pragma unroll
    for (int e0 = 0; e0 < kD; e0 += 8) {
        float f[8];
        load8f(row + e0, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) xf[e0 + e] = f[e];
    }
}

// x . r over the kD values of a row, in order from 0; x(e) gives value e of the
// row (registers or LDS), r[e * rstride] the projection's value e (LDS).  The
// projection's values are read 32 at a time ahead of their multiply-adds.
template <class X>
__device__ __forceinline__ double proj_chain(X&& x, const float* r, int rstride) {
    double z = 0.0;
#pragma unroll
    for (int e0 = 0; e0 < kD; e0 += 32) {
        float rv[32], xv[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            rv[k] = r[(e0 + k) * rstride];
            xv[k] = x(e0 + k);
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) z = __fma_rn((double)xv[k], (double)rv[k], z);
    }
    return z;
}

}  // namespace lcda
