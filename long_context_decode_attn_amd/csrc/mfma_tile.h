// mfma_tile.h - the 16-row x 32-token attention tile on CDNA4 matrix cores
// (v_mfma_f32_16x16x32_bf16), shared by the split-KV kernels.
//
// A wavefront owns 16*NT query rows and consumes a 32-token block of K/V held
// in registers (BlockRegs, the layout load_block / the LDS ring produce):
// S^T = K Q^T with K rows as the A operand, then O += P V with P already in
// A-operand layout in the lane that computed it (tokens are permuted inside the
// block, V is read in the same order and transposed in registers with
// v_perm_b32), split into bf16 hi + lo halves.  Online softmax in base 2 of
// "Nectar: Neural Estimation of Cached-Token Attention via Regression", Eq.
// (3.1): m, l and acc per row, with a lazy rescale (the running max only moves
// when a block max exceeds it by more than 2^8).
#pragma once

#include "common.h"

namespace lcda {

constexpr int kWaves = 4;
constexpr int kBlock = 32;
constexpr float kLazy = 8.0f;

template <int NT>
struct MfmaSmem {
    float o[kWaves][16 * NT][kD];
    float2 ml[kWaves][16 * NT];
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Position inside the 32-token block of the e-th k element held by lane group j.
__device__ __forceinline__ int tok_of(int j, int e) { return (e < 4) ? (4 * j + e) : (16 + 4 * j + e - 4); }

// p ~= hi + lo with hi = bf16(p) (nearest-even) and lo = bf16(p - hi).
__device__ __forceinline__ void split_hi_lo(const float (&p)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        f32x2 x = {p[e], p[e + 1]};
        bf16x2 h = __builtin_convertvector(x, bf16x2);
        f32x2 back = __builtin_convertvector(h, f32x2);
        bf16x2 l = __builtin_convertvector(x - back, bf16x2);
        hi[e] = h[0];
        hi[e + 1] = h[1];
        lo[e] = l[0];
        lo[e + 1] = l[1];
    }
}

struct BlockRegs {
    u32x4 k[2][4];  // [16-token half][32-wide d chunk]
    u32x4 v[8];     // [k element e]: 8 d values of token tok_of(j, e)
};


template <int NT>
struct WaveState {
    bf16x8 q[NT][4];
    f32x4 o[NT][8];
    float m[NT];
    float l[NT];
};

// valid: tokens of the block that exist (the rest are masked); col_ok: bit rt
// set = this lane's query row (c16) of row tile rt sees the block at all (a
// clear bit masks every token of that row).
// The logits stay unscaled up to the exponent: the row max of s*scale is
// scale times the max of s (scale > 0), and p = exp2(fma(s, scale, -m)).
template <int NT>
__device__ __forceinline__ void compute_block(WaveState<NT>& st, const BlockRegs& r, int valid, float scale, int j,
                                              int c16, int col_ok = -1) {
    // V operand: column n = c16 of d-block nb is d = 8*c16 + nb; k element e is token tok_of(j, e).
    bf16x8 vb[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
        const uint32_t sel = (nb & 1) ? 0x07060302u : 0x05040100u;
        u32x4 x;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
            x[qd] = __builtin_amdgcn_perm(r.v[2 * qd + 1][nb >> 1], r.v[2 * qd][nb >> 1], sel);
        vb[nb] = as_bf16x8(x);
    }
    // Scores: s[rt][tb][i] is token 16*tb + 4*j + i of the block, row 16*rt + c16.
    f32x4 s[NT][2];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.k[tb][c]), st.q[rt][c], acc, 0, 0, 0);
            s[rt][tb] = acc;
        }
    // Masking only where some token is missing or some row does not see the
    // block (a uniform branch around it).
    constexpr int kAll = (1 << NT) - 1;
    const int ok = col_ok & kAll;
    if (__builtin_amdgcn_readfirstlane(valid) < kBlock || __ballot(ok != kAll) != 0) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * tb + 4 * j + i >= valid || !((ok >> rt) & 1)) s[rt][tb][i] = -INFINITY;
    }
    float bm[NT];
    bool need = false;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[rt][tb][i]);
        mx = max_xor32(max_xor16(mx)) * scale;
        bm[rt] = mx;
        need |= (mx > st.m[rt] + kLazy);
    }
    if (__ballot(need)) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            const float mnew = fmaxf(st.m[rt], bm[rt]);
            const float alpha = fast_exp2(st.m[rt] - mnew);
            st.m[rt] = mnew;
            st.l[rt] *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * j + i, 64);  // row 4j+i lives in lane 4j+i
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) st.o[rt][nb][i] *= ai;
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        const float nm = -st.m[rt];
        float p[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[4 * tb + i] = fast_exp2(fmaf(s[rt][tb][i], scale, nm));
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ps += p[e];
        st.l[rt] += ps;
        bf16x8 hi, lo;
        split_hi_lo(p, hi, lo);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            st.o[rt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, vb[nb], st.o[rt][nb], 0, 0, 0);
            st.o[rt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, vb[nb], st.o[rt][nb], 0, 0, 0);
        }
    }
}

}  // namespace lcda
