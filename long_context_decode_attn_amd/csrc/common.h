// common.h - device types and helpers shared by the gfx950 kernels of liblcda.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;                       // head dimension (fixed)
constexpr float kLog2e = 1.4426950408889634f; // log2(e)
constexpr float kLn2 = 0.6931471805599453f;   // ln(2)
// Finite stand-in for "no token seen yet": exp2(kNoMax - m) is 0 for any real
// m, and kNoMax - kNoMax is 0 (no NaN), unlike -inf.
constexpr float kNoMax = -1.0e30f;

// One partial softmax state per (query row, slot): m = max of the scaled
// logits s*log2(e)/sqrt(d) seen, l = sum of exp2(scaled - m), acc[d] = sum of
// exp2(scaled - m) * v.  l == 0 marks an empty slot.
struct Partials {
    float2* ml;   // [rows][slots]
    float* acc;   // [rows][slots][kD]
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-lane butterfly sum (lanes l, l^1, l^2, l^4, l^8 of one row of 16).
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace lcda
