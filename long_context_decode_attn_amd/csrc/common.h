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

// Final value of one (row, column) from the merged partial state (M, L, acc)
// of all its tokens, merged with the optional virtual pair (alpha_in, a_in) -
// given here as values already read (virt = the pair is present and
// alpha_in > -inf) - exactly as the combine pass does; used when a row has a
// single split.  bhq = b*Hq + hq.
template <typename Args>
__device__ __forceinline__ void finish_row(const Args& a, int64_t bhq, int c, float M, float L, float acc,
                                           bool virt, float alpha_in, float a_in) {
    const bool has = L > 0.f;
    if (!has && !virt) {
        a.out[bhq * kD + c] = 0.f;
        if (a.alpha && c == 0) a.alpha[bhq] = -INFINITY;
        return;
    }
    const float mv = virt ? alpha_in * kLog2e : kNoMax;
    const float Mx = fmaxf(has ? M : kNoMax, mv);
    const float w = has ? fast_exp2(M - Mx) : 0.f;
    const float wv = virt ? fast_exp2(mv - Mx) : 0.f;
    const float Lx = w * L + wv;
    float x = w * acc;
    if (virt) x += wv * a_in;
    a.out[bhq * kD + c] = x * (1.f / Lx);
    if (a.alpha && c == 0) a.alpha[bhq] = (Mx + log2f(Lx)) * kLn2;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// s_waitcnt vmcnt(0): wait for every vector-memory load issued so far (gfx9
// encoding: vmcnt = 0, expcnt and lgkmcnt left at their maxima).  Used to drain
// a kernel prologue so that a software-pipelined loop starts from a state in
// which only its own block loads are outstanding.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16-byte load marked nontemporal (streamed once; do not keep in cache).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <bool NT>
__device__ __forceinline__ u32x4 ld16s(const void* p) {
    return NT ? ld16_nt(p) : ld16(p);
}

}  // namespace lcda
