// sig_topk_wide.hip - SCORE + TOPK over codes of W 32-bit words (b = 32 W bits,
// W = 1, 2, 4, 8 or 16): the distance popcount(h_i XOR h_q) of "HashAttention:
// Semantic Sparsity for Faster Inference", slide "A 32-bit signature makes
// scoring cheap", Eq. (2), summed over the words, so it runs from 0 to b.  The
// selection is the 32-bit one (slides "Only selection is approximate; selected
// KV stay in full form" and "Token-level sparsity still needs a careful
// kernel"): the m positions of smallest distance over all n positions, ties to
// the lower position, united with the windows [0, n_sink) and [n - n_recent, n),
// ascending, padded with -1.  Wider codes are the ones the pages' code-width
// sweep scores (slide with Table 6, 64 to 512 bits).
//
// One workgroup of 16 wavefronts per query head (row), in three phases:
//   1. every position's distance, kept in the workspace (u16), and a b+1-bin
//      histogram, one copy per wavefront in LDS;
//   2. the threshold t (the first bin whose prefix reaches m) and the quota of
//      ties at t the top m takes;
//   3. ordered compaction in tiles of 16,384 positions (16 consecutive per
//      thread): one wavefront-plus-LDS scan per tile of the selected and the
//      tie counts, packed in the two halves of a word, places every position.
// This is the plain form: a head's G query heads each read the key codes.

#include "common.h"
#include "internal.h"
#include "sparse.h"

namespace lcda {
namespace {

constexpr int kWThreads = 1024;
constexpr int kWWaves = kWThreads / 64;
constexpr int kWPer = 16;                       // positions per thread and tile
constexpr int kWTile = kWThreads * kWPer;

__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

template <int W>
__global__ __launch_bounds__(kWThreads) void k_topk_wide(WideArgs a) {
    constexpr int kBinsW = 32 * W + 1;
    __shared__ uint32_t hist[kWWaves][kBinsW];
    __shared__ uint32_t s_tot[kBinsW];
    __shared__ uint32_t s_wave[kWWaves];
    __shared__ int s_t;
    __shared__ uint32_t s_quota;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t row = blockIdx.x;
    const int b = (int)(row / a.Hq), hq = (int)(row % a.Hq), h = hq / a.G;
    const int64_t n = a.n;
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * n * W;
    uint16_t* dist = a.dist + row * n;
    uint32_t q[W];
#pragma unroll
    for (int k = 0; k < W; ++k) q[k] = a.q_sigs[row * W + k];
    for (int k = tid; k < kWWaves * kBinsW; k += kWThreads) (&hist[0][0])[k] = 0u;
    __syncthreads();

    // 1. distances and per-wavefront histograms
    for (int64_t i = tid; i < n; i += kWThreads) {
        const uint32_t* kp = ks + i * W;
        uint32_t d = 0;
        if constexpr (W % 4 == 0) {
#pragma unroll
            for (int k = 0; k < W; k += 4) {
                const u32x4 v = ld16(kp + k);
#pragma unroll
                for (int e = 0; e < 4; ++e) d += (uint32_t)__builtin_popcount(v[e] ^ q[k + e]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < W; ++k) d += (uint32_t)__builtin_popcount(kp[k] ^ q[k]);
        }
        dist[i] = (uint16_t)d;
        if (a.scores) a.scores[row * n + i] = (int16_t)(-(int)d);
        __hip_atomic_fetch_add(&hist[w][d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    for (int k = tid; k < kBinsW; k += kWThreads) {
        uint32_t sum = 0;
#pragma unroll
        for (int ww = 0; ww < kWWaves; ++ww) sum += hist[ww][k];
        s_tot[k] = sum;
    }
    __syncthreads();

    // 2. threshold and quota (wavefront 0; lane l owns bins l*per .. l*per + per - 1)
    const uint32_t meff = (uint32_t)min(a.m, n);
    if (w == 0) {
        constexpr int per = (kBinsW + 63) / 64;
        uint32_t c[per], sum = 0;
#pragma unroll
        for (int k = 0; k < per; ++k) {
            const int bin = lane * per + k;
            c[k] = bin < kBinsW ? s_tot[bin] : 0u;
            sum += c[k];
        }
        const uint32_t incl = wave_scan_incl(sum);
        const uint32_t before = incl - sum;
        // the lane whose range first reaches meff holds t
        const uint64_t reach = __ballot(meff > 0 && incl >= meff);
        if (lane == 0 && meff == 0) {
            s_t = -1;
            s_quota = 0u;
        }
        if (reach && lane == (int)__builtin_ctzll(reach)) {
            uint32_t run = before;
#pragma unroll
            for (int k = 0; k < per; ++k) {
                if (run + c[k] >= meff) {
                    s_t = lane * per + k;
                    s_quota = meff - run;
                    break;
                }
                run += c[k];
            }
        }
    }
    __syncthreads();
    const int t = s_t;
    const uint32_t quota = s_quota;
    const int64_t s_end = min(a.n_sink, n);
    const int64_t r_beg = max((int64_t)0, n - a.n_recent);

    // 3. ordered compaction: packed counts (selected in the low half, ties at t in the high half)
    int32_t* out = a.idx + row * a.cap;
    uint32_t ties_run = 0, sel_run = 0;   // over the tiles before, uniform
    for (int64_t t0 = 0; t0 < n; t0 += kWTile) {
        const int64_t p0 = t0 + (int64_t)tid * kWPer;
        uint32_t dd[kWPer];
#pragma unroll
        for (int k = 0; k < kWPer; ++k) dd[k] = p0 + k < n ? (uint32_t)dist[p0 + k] : 0xFFFFu;
        uint32_t tiem = 0;
#pragma unroll
        for (int k = 0; k < kWPer; ++k) tiem |= ((int)dd[k] == t ? 1u : 0u) << k;
        const uint32_t nt = (uint32_t)__builtin_popcount(tiem);
        // ties before this thread
        const uint32_t ti = wave_scan_incl(nt);
        if (lane == 63) s_wave[w] = ti;
        __syncthreads();
        uint32_t tb = ties_run + ti - nt, tall = 0;
#pragma unroll
        for (int ww = 0; ww < kWWaves; ++ww) {
            tb += ww < w ? s_wave[ww] : 0u;
            tall += s_wave[ww];
        }
        __syncthreads();
        uint32_t selm = 0;
#pragma unroll
        for (int k = 0; k < kWPer; ++k) {
            const int64_t p = p0 + k;
            const bool tie = (tiem >> k) & 1u;
            const uint32_t rank = tb + (uint32_t)__builtin_popcount(tiem & ((1u << k) - 1u));
            const bool top = (int)dd[k] < t || (tie && rank < quota);
            const bool sel = p < n && (top || p < s_end || p >= r_beg);
            selm |= (sel ? 1u : 0u) << k;
        }
        const uint32_t ns = (uint32_t)__builtin_popcount(selm);
        const uint32_t si = wave_scan_incl(ns);
        if (lane == 63) s_wave[w] = si;
        __syncthreads();
        uint32_t sb = sel_run + si - ns, sall = 0;
#pragma unroll
        for (int ww = 0; ww < kWWaves; ++ww) {
            sb += ww < w ? s_wave[ww] : 0u;
            sall += s_wave[ww];
        }
        __syncthreads();
        uint32_t m = selm;
        while (m) {
            const int k = __builtin_ctz(m);
            if ((int64_t)sb < a.cap) out[sb] = (int32_t)(p0 + k);
            ++sb;
            m &= m - 1u;
        }
        ties_run += tall;
        sel_run += sall;
    }
    if (tid == 0) a.count[row] = (int32_t)min((int64_t)sel_run, a.cap);
    for (int64_t i = (int64_t)sel_run + tid; i < a.cap; i += kWThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk_wide(const WideArgs& a, hipStream_t st) {
    if (a.B <= 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)a.B * a.Hq)), block(kWThreads);
    switch (a.W) {
        case 1: hipLaunchKernelGGL(k_topk_wide<1>, grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_topk_wide<2>, grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL(k_topk_wide<4>, grid, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL(k_topk_wide<8>, grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL(k_topk_wide<16>, grid, block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lcda
