// sig_topk.hip - HashAttention SCORE + TOPK over 32-bit signatures.
//
// SCORE(k_i, q) = -popcount(h_i XOR h_q) ("HashAttention: Semantic Sparsity
// for Faster Inference", slide "A 32-bit signature makes scoring cheap",
// Eq. (2)); TOPK keeps the m positions of smallest distance, ties to the lower
// position, united with the first n_sink and last n_recent positions, in
// ascending order.
//
// Distances take only 33 values, so the top m is fixed by a threshold pair
// (t, p): position i is in the top m iff (d_i, i) < (t, p) in lexicographic
// order, i.e. the 64-bit key (d_i << 32 | i) is below K = (t << 32 | p).
// Three kernels, each reading the signatures of a KV head once for all G query
// heads of its group:
//   1. k_sig_hist    - per chunk of kChunk positions and query head, the
//                      33-bin histogram of distances (lane-private LDS counters:
//                      no two lanes ever touch one LDS word, so no conflicts).
//   2. k_topk_select - per query head: global histogram -> t and the tie quota;
//                      the chunk holding the last tie taken is scanned for the
//                      position p; the windows add the positions they hold
//                      outside the top m; per-chunk output offsets by an
//                      exclusive scan; count and the -1 padding are written.
//   3. k_sig_compact - per chunk: recompute the keys (the signatures are still
//                      cache-resident), flag top-m or window positions and write
//                      them in order with ballot / mbcnt prefix counts.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

constexpr int kChunk = 4096;   // positions per chunk
constexpr int kMaxG = 8;       // query heads per KV head handled by one pass
constexpr int kBins = 33;

__device__ __forceinline__ uint64_t sel_key(uint32_t d, int64_t i) {
    return ((uint64_t)d << 32) | (uint64_t)(uint32_t)i;
}

// ---- 1. histogram -----------------------------------------------------------
template <int MAXG, bool VEC>
__global__ __launch_bounds__(64) void k_sig_hist(TopkArgs a) {
    __shared__ uint32_t cnt[MAXG * kBins * 64];   // [g][bin][lane]
    const int lane = threadIdx.x;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int G = a.G;
    for (int k = lane; k < G * kBins * 64; k += 64) cnt[k] = 0;   // own column only

    uint32_t qs[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) qs[g] = g < G ? a.q_sigs[(int64_t)b * a.Hq + h * G + g] : 0u;

    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int64_t beg = (int64_t)c * kChunk;
    const int64_t end = min(a.n, beg + (int64_t)kChunk);
    int8_t* sc = a.scores ? a.scores + ((int64_t)b * a.Hq + h * G) * a.n : nullptr;

    for (int64_t i = beg + 4 * lane; i < end; i += 256) {
        uint32_t x[4];
        if (VEC && i + 3 < end) {
            const u32x4 v = ld16(ks + i);
            x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (i + e < end) ? ks[i + e] : 0u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (i + e >= end) break;
#pragma unroll
            for (int g = 0; g < MAXG; ++g) {
                if (g >= G) break;
                const uint32_t d = __builtin_popcount(x[e] ^ qs[g]);
                __hip_atomic_fetch_add(&cnt[(g * kBins + d) * 64 + lane], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                if (sc) sc[(int64_t)g * a.n + i + e] = (int8_t)(-(int)d);
            }
        }
    }
    __syncthreads();
    // Sum the 64 lane columns of each (g, bin) row; lane l starts at column l so
    // the 64 lanes of a read hit 64 different banks.
    for (int row = lane; row < G * kBins; row += 64) {
        uint32_t s = 0;
        for (int k = 0; k < 64; ++k) s += cnt[row * 64 + ((k + lane) & 63)];
        const int g = row / kBins, bin = row % kBins;
        a.hist[(((int64_t)b * a.Hq + h * G + g) * a.chunks + c) * kBins + bin] = s;
    }
}

// ---- block-wide exclusive scan (256 threads) ----------------------------------
__device__ int64_t block_exclusive_scan(int64_t x, int64_t* total, int64_t* sh /*[4+1]*/) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int64_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    int64_t base = 0, all = 0;
    for (int ww = 0; ww < 4; ++ww) {
        if (ww < w) base += sh[ww];
        all += sh[ww];
    }
    __syncthreads();
    *total = all;
    return base + inc - x;
}

// ---- 2. threshold, windows, offsets -----------------------------------------
__global__ __launch_bounds__(256) void k_topk_select(TopkArgs a) {
    __shared__ uint32_t H[kBins];
    __shared__ int64_t scan_sh[4];
    __shared__ int s_t;
    __shared__ int64_t s_quota, s_cstar, s_rank, s_pt;
    const int tid = threadIdx.x;
    const int hq = blockIdx.x, b = blockIdx.y;
    const int h = hq / a.G;
    const int64_t row = (int64_t)b * a.Hq + hq;
    const uint32_t* hist = a.hist + row * a.chunks * kBins;
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const uint32_t qsig = a.q_sigs[row];
    const int C = a.chunks;

    if (tid < kBins) H[tid] = 0;
    __syncthreads();
    for (int e = tid; e < C * kBins; e += 256) atomicAdd(&H[e % kBins], hist[e]);
    __syncthreads();
    if (tid == 0) {
        const int64_t meff = min(a.m, a.n);
        int t = -1;
        int64_t cum = 0, quota = 0;
        if (meff > 0) {
            for (int d = 0; d < kBins; ++d) {
                if (cum + (int64_t)H[d] >= meff) {
                    t = d;
                    quota = meff - cum;
                    break;
                }
                cum += H[d];
            }
        }
        s_t = t;
        s_quota = quota;
        s_cstar = -1;
        s_rank = 0;
        s_pt = -1;
    }
    __syncthreads();
    const int t = s_t;
    const int64_t quota = s_quota;

    // Chunk c* holding the quota-th tie (distance t), and its rank inside c*.
    if (t >= 0) {
        int64_t carry = 0;
        for (int c0 = 0; c0 < C; c0 += 256) {
            const int c = c0 + tid;
            const int64_t eq = c < C ? hist[(int64_t)c * kBins + t] : 0;
            int64_t tot;
            const int64_t pre = carry + block_exclusive_scan(eq, &tot, scan_sh);
            if (c < C && pre < quota && quota <= pre + eq) {
                s_cstar = c;
                s_rank = quota - pre;   // 1-based rank inside chunk c
            }
            carry += tot;
        }
        __syncthreads();
        // Position of that tie: 256 threads x 16 consecutive positions of c*.
        const int64_t cs = s_cstar;
        const int64_t beg = cs * kChunk;
        const int64_t my = beg + (int64_t)tid * (kChunk / 256);
        const int64_t my_end = min(a.n, my + (int64_t)(kChunk / 256));
        int64_t cnt = 0;
        if (cs >= 0)
            for (int64_t i = my; i < my_end; ++i) cnt += (__builtin_popcount(ks[i] ^ qsig) == (uint32_t)t);
        int64_t tot;
        const int64_t pre = block_exclusive_scan(cnt, &tot, scan_sh);
        const int64_t want = s_rank;
        if (cs >= 0 && pre < want && want <= pre + cnt) {
            int64_t r = pre;
            for (int64_t i = my; i < my_end; ++i) {
                if (__builtin_popcount(ks[i] ^ qsig) == (uint32_t)t && ++r == want) {
                    s_pt = i;
                    break;
                }
            }
        }
        __syncthreads();
    }
    const int64_t cstar = s_cstar, rank_in = s_rank;
    const uint64_t K = (t < 0) ? 0ull : sel_key((uint32_t)t, s_pt + 1);

    // Per-chunk selected counts -> exclusive offsets.
    const int64_t n = a.n, s_end = min(a.n_sink, n), r_beg = max((int64_t)0, n - a.n_recent);
    int64_t carry = 0;
    for (int c0 = 0; c0 < C; c0 += 256) {
        const int c = c0 + tid;
        int64_t cnt = 0;
        if (c < C) {
            const uint32_t* hc = hist + (int64_t)c * kBins;
            for (int d = 0; d < t; ++d) cnt += hc[d];
            if (t >= 0) cnt += (c < cstar) ? (int64_t)hc[t] : (c == cstar ? rank_in : 0);
            // window positions of this chunk that are not already in the top m
            const int64_t cb = (int64_t)c * kChunk, ce = min(n, cb + (int64_t)kChunk);
            for (int64_t i = cb; i < min(ce, s_end); ++i)
                cnt += sel_key(__builtin_popcount(ks[i] ^ qsig), i) >= K;
            for (int64_t i = max(cb, max(r_beg, s_end)); i < ce; ++i)
                cnt += sel_key(__builtin_popcount(ks[i] ^ qsig), i) >= K;
        }
        int64_t tot;
        const int64_t off = carry + block_exclusive_scan(cnt, &tot, scan_sh);
        if (c < C) a.chunk_info[row * C + c] = (int32_t)off;
        carry += tot;
    }
    if (tid == 0) {
        a.count[row] = (int32_t)carry;
        reinterpret_cast<uint64_t*>(a.head_info)[row] = K;
    }
    for (int64_t i = carry + tid; i < a.cap; i += 256) a.idx[row * a.cap + i] = -1;
}

// ---- 3. ordered compaction ----------------------------------------------------
__global__ __launch_bounds__(64) void k_sig_compact(TopkArgs a) {
    const int lane = threadIdx.x;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int G = a.G;
    const int64_t row0 = (int64_t)b * a.Hq + h * G;
    uint32_t qs[kMaxG];
    uint64_t K[kMaxG];
    int64_t off[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
        if (g < G) {
            qs[g] = a.q_sigs[row0 + g];
            K[g] = reinterpret_cast<const uint64_t*>(a.head_info)[row0 + g];
            off[g] = a.chunk_info[(row0 + g) * a.chunks + c];
        } else {
            qs[g] = 0;
            K[g] = 0;
            off[g] = 0;
        }
    }
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int64_t beg = (int64_t)c * kChunk;
    const int64_t end = min(a.n, beg + (int64_t)kChunk);
    const int64_t s_end = min(a.n_sink, a.n), r_beg = max((int64_t)0, a.n - a.n_recent);
    const uint64_t below = (1ull << lane) - 1ull;

    for (int64_t base = beg; base < end; base += 256) {
        uint32_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + 64 * u + lane;
            x[u] = i < end ? ks[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + 64 * u + lane;
            const bool valid = i < end;
            const bool win = i < s_end || i >= r_beg;
#pragma unroll
            for (int g = 0; g < kMaxG; ++g) {
                if (g >= G) break;
                const uint32_t d = __builtin_popcount(x[u] ^ qs[g]);
                const bool sel = valid && (win || sel_key(d, i) < K[g]);
                const uint64_t mask = __ballot(sel);
                if (mask) {
                    const int64_t pos = off[g] + __popcll(mask & below);
                    if (sel && pos < a.cap) a.idx[(row0 + g) * a.cap + pos] = (int32_t)i;
                    off[g] += __popcll(mask);
                }
            }
        }
    }
}

}  // namespace

int topk_chunk_len(int64_t) { return kChunk; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    if (a.B <= 0) return hipSuccess;
    if (a.G > kMaxG) return hipErrorInvalidValue;
    const dim3 gc(a.chunks, a.Hkv, a.B);
    hipError_t e;
    if (a.chunks > 0) {
        const bool vec = a.n % 4 == 0;
        if (a.G <= 4) {
            if (vec) hipLaunchKernelGGL((k_sig_hist<4, true>), gc, dim3(64), 0, st, a);
            else hipLaunchKernelGGL((k_sig_hist<4, false>), gc, dim3(64), 0, st, a);
        } else {
            if (vec) hipLaunchKernelGGL((k_sig_hist<8, true>), gc, dim3(64), 0, st, a);
            else hipLaunchKernelGGL((k_sig_hist<8, false>), gc, dim3(64), 0, st, a);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_select, dim3(a.Hq, a.B), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.chunks > 0) hipLaunchKernelGGL(k_sig_compact, gc, dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcda
