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
constexpr int kRsrcWord3 = 0x00020000;        // gfx9 raw buffer resource: 32-bit data format, no swizzle
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

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r + 15), returned in all
// of them: swaps of neighbours and of pairs inside each group of four
// (quad_perm [1,0,3,2] and [2,3,0,1]), then rotations of the row by 4 and by 8.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum16(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_mov<0x124>(x);   // row_ror:4
    x += dpp_mov<0x128>(x);   // row_ror:8
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

// s_waitcnt vmcnt(0): wait for every vector-memory access issued so far to
// complete (gfx9 encoding: vmcnt = 0, expcnt and lgkmcnt left at their
// maxima; on gfx9 vmcnt counts stores as well as loads).  Drains a kernel
// prologue so that a software-pipelined loop starts with only its own block
// loads outstanding, and waits for stores to be acknowledged.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Reductions over lanes {l, l ^ 16} and {l, l ^ 32} without LDS: a
// v_permlane16_swap (v_permlane32_swap) of two copies of x leaves, in every
// lane l, the pair x[l & ~16], x[l | 16] (x[l & ~32], x[l | 32]) in the two
// registers.  Issued as inline asm on two distinct registers: the compiler's
// intrinsic for it folds the swap of a value with itself into a no-op.  The
// s_nop 1 gives the two wait states the swap needs after the VALU writes of
// its operands.
__device__ __forceinline__ void swap16(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_xor16(float x) {
    float a = x, b = x;
    swap16(a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float max_xor32(float x) {
    float a = x, b = x;
    swap32(a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor16(float x) {
    float a = x, b = x;
    swap16(a, b);
    return a + b;
}
__device__ __forceinline__ float sum_xor32(float x) {
    float a = x, b = x;
    swap32(a, b);
    return a + b;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Partial states cross workgroups (and XCDs, whose L2 caches are not kept
// coherent with each other) through device-scope stores and loads: a store
// with device scope is written through to the device's coherence point before
// it is acknowledged, and a load with device scope reads from there.  Only
// these values are published, so no whole-cache write-back or invalidate is
// needed.
__device__ __forceinline__ void store_dev(float* p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(float2* p, float2 x) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       __builtin_bit_cast(unsigned long long, x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint32_t* p, uint32_t x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_dev_u32(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_dev_u64(const void* p) {   // 8-byte aligned
    return __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 load_dev2(const float* p) {   // two adjacent floats, 8-byte aligned
    return __builtin_bit_cast(f32x2, __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Arrival counter words hold a 52-bit tag above a 12-bit count of arrivals
// (targets up to 4,095; the launchers never exceed 2,048).
constexpr int kCtrCountBits = 12;
constexpr unsigned long long kCtrCountMask = (1ull << kCtrCountBits) - 1ull;
constexpr int kCtrMaxTarget = (int)kCtrCountMask;

// Tag of the arrival counter at address c, in the word's upper 52 bits: a hash
// of the address (the SplitMix64 finalizer), so that a counter word is
// recognised as one this library left (tag, 0) and anything else (a fresh
// workspace, other data) is not.  Bytes that were never a counter hold a given
// tag with probability 2^-52.
__device__ __forceinline__ unsigned long long ctr_tag(const unsigned long long* c) {
    unsigned long long x = (unsigned long long)(uintptr_t)c;
    x ^= x >> 30;
    x *= 0xBF58476D1CE4E5B9ull;
    x ^= x >> 27;
    x *= 0x94D049BB133111EBull;
    x ^= x >> 31;
    return x & ~kCtrCountMask;
}

// One arrival at counter c, made by one thread once the workgroup's published
// stores are acknowledged: returns the number of arrivals so far, this one
// included, and restores (tag, 0) when that is `target`.  Normally one
// fetch-add; a counter word without its tag (never used, or overwritten) is
// replaced by (tag, 1) with a compare-exchange by the first arrival to find it
// so, and the others then count on the valid word (the exchange loop ends once
// any of them has installed it).
__device__ __forceinline__ uint32_t arrive_one(unsigned long long* c, uint32_t target) {
    const unsigned long long valid0 = ctr_tag(c);
    unsigned long long old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t count;
    if ((old & ~kCtrCountMask) == valid0) {
        count = (uint32_t)(old & kCtrCountMask) + 1u;
    } else {
        unsigned long long cur = old + 1ull;
        while (true) {
            if ((cur & ~kCtrCountMask) == valid0) {
                old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                count = (uint32_t)(old & kCtrCountMask) + 1u;
                break;
            }
            if (__hip_atomic_compare_exchange_strong(c, &cur, valid0 | 1ull, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)) {
                count = 1u;
                break;
            }
        }
    }
    if (count == target) __hip_atomic_store(c, valid0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return count;
}

// Arrival of one workgroup at counter c, after every thread wrote what it
// publishes with device-scope stores: returns true, in every thread, in the
// last of `target` workgroups to arrive.  The counter holds (tag, arrivals);
// between calls it is (tag, 0), which the last arrival restores (see
// arrive_one).
__device__ __forceinline__ bool arrive_count(unsigned long long* c, uint32_t target, int* s_flag) {
    wait_vm_all();    // this thread's device-scope stores are acknowledged
    __syncthreads();  // ... in every thread of the workgroup
    if (threadIdx.x == 0) *s_flag = arrive_one(c, target) == target ? 1 : 0;
    __syncthreads();
    return *s_flag != 0;
}

// The split pass's arrival: unit `unit` has a.splits workgroups.
template <class Args>
__device__ __forceinline__ bool arrive_last(const Args& a, int64_t unit, int* s_flag) {
    return arrive_count(a.ctr + unit, (uint32_t)a.splits, s_flag);
}

// Exactly kFewSplits splits (the split count of a full-chip launch over one
// batch item's 8 KV heads): every load of the row (its (m, l) pairs, its
// partial vectors and the virtual pair) is requested at once, at offsets
// known at compile time, so the merge waits for one memory round trip; the
// sums run in the same order as in combine_row's general loop.
constexpr int kFewSplits = 32;

template <class Args>
__device__ __forceinline__ void combine_row_few(const Args& a, int64_t bhq, int lane) {
    const int S = a.splits;
    const float* ml = reinterpret_cast<const float*>(a.ml + bhq * S);
    const float* acc = a.acc + bhq * S * kD + 2 * lane;
    const f32x2 x = load_dev2(ml + 2 * (lane & (kFewSplits - 1)));   // lanes at or past S are ignored
    f32x2 v[kFewSplits];
#pragma unroll
    for (int s = 0; s < kFewSplits; ++s) v[s] = load_dev2(acc + s * kD);
    const float al_in = a.alpha_in != nullptr ? a.alpha_in[bhq] : -INFINITY;
    const f32x2 a_in = a.alpha_in != nullptr ? *reinterpret_cast<const f32x2*>(a.a_in + bhq * kD + 2 * lane)
                                             : f32x2{0.f, 0.f};
    const bool has = lane < S && x.y > 0.f;
    const bool virt = al_in > -INFINITY;
    if (!__any(has) && !virt) {
        *reinterpret_cast<f32x2*>(a.out + bhq * kD + 2 * lane) = f32x2{0.f, 0.f};
        if (a.alpha && lane == 0) a.alpha[bhq] = -INFINITY;
        return;
    }
    const float mv = virt ? al_in * kLog2e : kNoMax;
    const float M = fmaxf(wave_max(has ? x.x : kNoMax), mv);
    const float w = has ? fast_exp2(x.x - M) : 0.f;
    f32x2 o = {0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kFewSplits; ++s) o += __shfl(w, s, 64) * v[s];   // split s's weight, in vector registers
    const float wv = virt ? fast_exp2(mv - M) : 0.f;
    const float L = wave_sum(w * x.y) + wv;
    if (virt) o += wv * a_in;
    *reinterpret_cast<f32x2*>(a.out + bhq * kD + 2 * lane) = o * (1.f / L);
    if (a.alpha && lane == 0) a.alpha[bhq] = (M + log2f(L)) * kLn2;
}

// One wave merges the a.splits partial states of query row bhq (and the
// optional virtual pair (a_in, alpha_in)) into out / alpha, as the combine
// pass does: M = max m_s, L = sum l_s 2^(m_s - M), A = sum acc_s 2^(m_s - M) / L.
// Partial states are read with device-scope loads.  Lane l owns output
// columns 2l, 2l + 1.
template <class Args>
__device__ __forceinline__ void combine_row(const Args& a, int64_t bhq, int lane) {
    const int S = a.splits;
    if (S == kFewSplits) {
        combine_row_few(a, bhq, lane);
        return;
    }
    const float* ml = reinterpret_cast<const float*>(a.ml + bhq * S);
    const float* acc = a.acc + bhq * S * kD + 2 * lane;
    float mloc = kNoMax;
    int anyl = 0;
    for (int s = lane; s < S; s += 64) {
        const f32x2 x = load_dev2(ml + 2 * s);
        if (x.y > 0.f) {
            mloc = fmaxf(mloc, x.x);
            anyl = 1;
        }
    }
    const bool virt = a.alpha_in != nullptr && a.alpha_in[bhq] > -INFINITY;
    if (!__any(anyl) && !virt) {
        *reinterpret_cast<f32x2*>(a.out + bhq * kD + 2 * lane) = f32x2{0.f, 0.f};
        if (a.alpha && lane == 0) a.alpha[bhq] = -INFINITY;
        return;
    }
    const float mv = virt ? a.alpha_in[bhq] * kLog2e : kNoMax;
    const float M = fmaxf(wave_max(mloc), mv);
    f32x2 o = {0.f, 0.f};
    float lsum = 0.f;
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int s = s0 + lane;
        const f32x2 x = s < S ? load_dev2(ml + 2 * s) : f32x2{kNoMax, 0.f};
        const float w = x.y > 0.f ? fast_exp2(x.x - M) : 0.f;
        lsum += w * x.y;
        const int wi_bits = __builtin_bit_cast(int, w);
        const int cnt = min(64, S - s0);
        const float* base = acc + (int64_t)s0 * kD;
        int i = 0;
        for (; i + 8 <= cnt; i += 8) {
            f32x2 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = load_dev2(base + (int64_t)(i + u) * kD);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                o += __builtin_bit_cast(float, __builtin_amdgcn_readlane(wi_bits, i + u)) * v[u];
        }
        for (; i < cnt; ++i)
            o += __builtin_bit_cast(float, __builtin_amdgcn_readlane(wi_bits, i)) * load_dev2(base + (int64_t)i * kD);
    }
    const float wv = virt ? fast_exp2(mv - M) : 0.f;
    const float L = wave_sum(lsum) + wv;
    if (virt) o += wv * *reinterpret_cast<const f32x2*>(a.a_in + bhq * kD + 2 * lane);
    *reinterpret_cast<f32x2*>(a.out + bhq * kD + 2 * lane) = o * (1.f / L);
    if (a.alpha && lane == 0) a.alpha[bhq] = (M + log2f(L)) * kLn2;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}


// 16-byte load marked nontemporal (streamed once; do not keep in cache).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <bool NT>
__device__ __forceinline__ u32x4 ld16s(const void* p) {
    return NT ? ld16_nt(p) : ld16(p);
}

}  // namespace lcda
