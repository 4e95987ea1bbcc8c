// sig_topk.hip - HashAttention SCORE + TOPK over 32-bit signatures.
//
// SCORE(k_i, q) = -popcount(h_i XOR h_q) ("HashAttention: Semantic Sparsity
// for Faster Inference", slide "A 32-bit signature makes scoring cheap",
// Eq. (2)); TOPK keeps the m positions of smallest distance, ties to the lower
// position, united with the first n_sink and last n_recent positions, in
// ascending order.
//
// Distances take only 33 values, so the top m is fixed by a threshold pair
// (t, p): position i is in the top m iff d_i < t, or d_i == t and i <= p.
// Three kernels; the two that scan signatures read each KV head's codes once
// for all G query heads of its group:
//   1. k_sig_hist    - per chunk of kChunk positions (one wavefront) and query
//                      head, the 33-bin histogram of distances.  Counts go to 16
//                      LDS copies (lane % 16), padded so lanes rarely collide.
//   2. k_topk_select - per query head: global histogram -> t and the tie quota;
//                      the chunk holding the last tie taken is scanned for p;
//                      chunks covered by a window are counted whole and the (at
//                      most two) chunks a window edge cuts are scanned; per-chunk
//                      output offsets by an exclusive scan; count and the -1
//                      padding are written.
//   3. k_sig_compact - per chunk: recompute the distances (the codes are still
//                      cache-resident), flag top-m or window positions and write
//                      them in order with ballot / mbcnt ranks.
// Each wavefront requests its whole chunk (4096 codes, 64 per lane) before
// using any of it.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

constexpr int kChunk = 4096;            // positions per chunk (one wavefront)
constexpr int kPerLane = kChunk / 64;   // codes per lane
constexpr int kMaxG = 8;                // query heads per KV head handled by one pass
constexpr int kBins = 33;
constexpr int kCopies = 16;             // LDS histogram copies (lane % 16)
constexpr int kBinStride = kCopies + 1; // words per bin (one pad word spreads banks)

// ---- 1. histogram -----------------------------------------------------------
// Lane l holds positions beg + 4*(l + 64*u) + e, u < kPerLane/4, e < 4.
// Positions fit in 32 bits (n <= INT32_MAX).  A full chunk runs without any
// per-position test; in the last, short chunk positions at or past the end
// count into a spare bin (kBins) that is never read.
template <int MAXG, bool VEC, bool SCORES>
__global__ __launch_bounds__(64) void k_sig_hist(TopkArgs a) {
    __shared__ uint32_t cnt[MAXG * (kBins + 1) * kBinStride];   // [g][bin][copy]
    const int lane = threadIdx.x;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int G = a.G;
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int beg = c * kChunk;
    const int end = (int)min(a.n, (int64_t)beg + kChunk);

    // Straight-line loads of clamped addresses (no branch between them, so
    // they are all in flight at once).
    u32x4 x[kPerLane / 4];
#pragma unroll
    for (int u = 0; u < kPerLane / 4; ++u) {
        const int i = beg + 4 * (lane + 64 * u);
        if (VEC) {
            x[u] = ld16(ks + min(i, end - 4));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[u][e] = ks[min(i + e, end - 1)];
        }
    }
    for (int k = lane; k < G * (kBins + 1) * kBinStride; k += 64) cnt[k] = 0;
    uint32_t qs[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) qs[g] = g < G ? a.q_sigs[(int64_t)b * a.Hq + h * G + g] : 0u;
    __syncthreads();

    uint32_t* my = cnt + lane % kCopies;
    const bool full = end - beg == kChunk;
#pragma unroll
    for (int u = 0; u < kPerLane / 4; ++u) {
        const int i = beg + 4 * (lane + 64 * u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = full || i + e < end;
#pragma unroll
            for (int g = 0; g < MAXG; ++g) {
                if (g < G) {
                    const uint32_t d = __builtin_popcount(x[u][e] ^ qs[g]);
                    const uint32_t bin = ok ? d : (uint32_t)kBins;
                    __hip_atomic_fetch_add(my + (g * (kBins + 1) + bin) * kBinStride, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
                    if (SCORES && ok) a.scores[((int64_t)b * a.Hq + h * G + g) * a.n + i + e] = (int8_t)(-(int)d);
                }
            }
        }
    }
    __syncthreads();
    for (int row = lane; row < G * kBins; row += 64) {
        const int g = row / kBins, bin = row % kBins;
        uint32_t sum = 0;
#pragma unroll
        for (int k = 0; k < kCopies; ++k) sum += cnt[(g * (kBins + 1) + bin) * kBinStride + k];
        a.hist[(((int64_t)b * a.Hq + h * G + g) * a.chunks + c) * kBins + bin] = sum;
    }
}

// ---- block-wide helpers (256 threads) -----------------------------------------
__device__ int64_t block_exclusive_scan(int64_t x, int64_t* total, int64_t* sh /*[4]*/) {
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

// The 16 codes [i0, i0 + 16) (zeros at and past end).
// The 16 codes [i0, i0 + 16) of a chunk [.., end) with end > 0; entries at or
// past end hold some in-range code and must be ignored by the caller.
__device__ __forceinline__ void load16(const uint32_t* ks, int64_t i0, int64_t end, bool vec, uint32_t (&x)[16]) {
    if (vec) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 v = ld16(ks + min(i0 + 4 * u, end - 4));
            x[4 * u] = v[0];
            x[4 * u + 1] = v[1];
            x[4 * u + 2] = v[2];
            x[4 * u + 3] = v[3];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = ks[min(i0 + e, end - 1)];
    }
}

// ---- 2. threshold, windows, offsets -----------------------------------------
constexpr int kSelHist = 8448;   // histogram words staged in LDS (256 chunks x 33 bins)

__global__ __launch_bounds__(256) void k_topk_select(TopkArgs a) {
    __shared__ uint32_t H[kBins];
    __shared__ uint32_t s_hist[kSelHist];
    __shared__ int64_t scan_sh[4];
    __shared__ int s_t;
    __shared__ int64_t s_quota, s_cstar, s_rank, s_pt, s_extra[2];
    const int tid = threadIdx.x;
    const int hq = blockIdx.x, b = blockIdx.y;
    const int h = hq / a.G;
    const int64_t row = (int64_t)b * a.Hq + hq;
    const uint32_t* hist = a.hist + row * a.chunks * kBins;
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const uint32_t qsig = a.q_sigs[row];
    const int C = a.chunks;
    const int64_t n = a.n;
    const bool vec = (n % 4) == 0;
    const bool staged = C * kBins <= kSelHist;

    // Windows [0, s_end) and [r_beg, n).  A chunk entirely inside a window is
    // selected whole; a chunk cut by a window edge gets the window positions it
    // holds outside the top m added (at most two such chunks).  Their codes are
    // requested first: they do not depend on the threshold.
    const int64_t s_end = min(a.n_sink, n);
    const int64_t r_beg = max(max((int64_t)0, n - a.n_recent), s_end);
    int64_t cut[2] = {-1, -1};
    if (s_end > 0 && s_end % kChunk != 0 && s_end < n) cut[0] = s_end / kChunk;
    if (r_beg < n && r_beg % kChunk != 0) cut[1] = r_beg / kChunk;
    if (cut[1] == cut[0]) cut[1] = -1;
    uint32_t xcut[2][16];
#pragma unroll
    for (int k = 0; k < 2; ++k)
        if (cut[k] >= 0) load16(ks, cut[k] * kChunk + 16 * tid, min(n, cut[k] * kChunk + (int64_t)kChunk), vec, xcut[k]);

    if (tid < kBins) H[tid] = 0;
    __syncthreads();
    for (int e = tid; e < C * kBins; e += 256) {
        const uint32_t v = hist[e];
        if (staged) s_hist[e] = v;
        atomicAdd(&H[e % kBins], v);
    }
    __syncthreads();
    auto hist_at = [&](int64_t c, int d) -> uint32_t {
        return staged ? s_hist[c * kBins + d] : hist[c * kBins + d];
    };
    if (tid == 0) {
        const int64_t meff = min(a.m, n);
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
        s_extra[0] = 0;
        s_extra[1] = 0;
    }
    __syncthreads();
    const int t = s_t;
    const int64_t quota = s_quota;

    // Chunk c* holding the quota-th tie (distance t), its rank there, and its position p.
    if (t >= 0) {
        int64_t carry = 0;
        for (int c0 = 0; c0 < C; c0 += 256) {
            const int c = c0 + tid;
            const int64_t eq = c < C ? hist_at(c, t) : 0;
            int64_t tot;
            const int64_t pre = carry + block_exclusive_scan(eq, &tot, scan_sh);
            if (c < C && pre < quota && quota <= pre + eq) {
                s_cstar = c;
                s_rank = quota - pre;   // 1-based rank inside chunk c
            }
            carry += tot;
        }
        __syncthreads();
        const int64_t cs = s_cstar;
        int64_t cnt = 0;
        uint32_t x[16];
        const int64_t i0 = cs * kChunk + 16 * tid;
        const int64_t cend = min(n, cs * kChunk + (int64_t)kChunk);
        if (cs >= 0) {
            load16(ks, i0, cend, vec, x);
#pragma unroll
            for (int e = 0; e < 16; ++e) cnt += (i0 + e < cend) && (__builtin_popcount(x[e] ^ qsig) == (uint32_t)t);
        }
        int64_t tot;
        const int64_t pre = block_exclusive_scan(cnt, &tot, scan_sh);
        const int64_t want = s_rank;
        if (cs >= 0 && pre < want && want <= pre + cnt) {
            int64_t r = pre;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (i0 + e < cend && __builtin_popcount(x[e] ^ qsig) == (uint32_t)t) {
                    ++r;
                    if (r == want) s_pt = i0 + e;
                }
            }
        }
        __syncthreads();
    }
    const int64_t cstar = s_cstar, rank_in = s_rank;
    const int64_t p1 = s_pt + 1;   // ties at positions < p1 are taken

#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (cut[k] < 0) continue;   // uniform across the block
        const int64_t cb = cut[k] * kChunk;
        const int64_t ce = min(n, cb + (int64_t)kChunk);
        const int64_t i0 = cb + 16 * tid;
        int64_t ex = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t i = i0 + e;
            const int d = __builtin_popcount(xcut[k][e] ^ qsig);
            const bool top = d < t || (d == t && i < p1);
            if (i < ce && (i < s_end || i >= r_beg) && !top) ++ex;
        }
        int64_t tot;
        block_exclusive_scan(ex, &tot, scan_sh);
        if (tid == 0) s_extra[k] = tot;
        __syncthreads();
    }

    int64_t carry = 0;
    for (int c0 = 0; c0 < C; c0 += 256) {
        const int c = c0 + tid;
        int64_t cnt = 0;
        if (c < C) {
            const int64_t cb = (int64_t)c * kChunk, ce = min(n, cb + (int64_t)kChunk);
            if (ce <= s_end || cb >= r_beg) {
                cnt = ce - cb;   // entirely inside a window
            } else {
                for (int d = 0; d < t; ++d) cnt += hist_at(c, d);
                if (t >= 0) cnt += (c < cstar) ? (int64_t)hist_at(c, t) : (c == cstar ? rank_in : 0);
                if (c == cut[0]) cnt += s_extra[0];
                if (c == cut[1]) cnt += s_extra[1];
            }
        }
        int64_t tot;
        const int64_t off = carry + block_exclusive_scan(cnt, &tot, scan_sh);
        if (c < C) a.chunk_info[row * C + c] = (int32_t)off;
        carry += tot;
    }
    if (tid == 0) {
        a.count[row] = (int32_t)carry;
        a.head_info[2 * row] = t;
        a.head_info[2 * row + 1] = (int32_t)p1;
    }
    for (int64_t i = carry + tid; i < a.cap; i += 256) a.idx[row * a.cap + i] = -1;
}

// ---- 3. ordered compaction ----------------------------------------------------
// The chunk is walked in 4 quarters of 1024 positions; in a quarter lane l holds
// positions base + l + 64*u, u < 16.  The next quarter is requested before the
// current one is processed.  Positions are 32-bit.
constexpr int kQuarter = kChunk / 4;

template <int MAXG>
struct CompactState {
    uint32_t qs[MAXG];
    int tt[MAXG];
    int p1[MAXG], off[MAXG];
};

__device__ __forceinline__ void load_quarter(uint32_t (&x)[16], const uint32_t* ks, int base, int end, int lane) {
#pragma unroll
    for (int u = 0; u < 16; ++u) x[u] = ks[min(base + lane + 64 * u, end - 1)];   // clamped; masked by the caller
}

template <int MAXG>
__device__ __forceinline__ void compact_quarter(const TopkArgs& a, CompactState<MAXG>& st, const uint32_t (&x)[16],
                                                int base, int end, int64_t row0, int s_end, int r_beg, int lane) {
    const int G = a.G;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int i = base + lane + 64 * u;
        const bool valid = i < end;
        const bool win = i < s_end || i >= r_beg;
#pragma unroll
        for (int g = 0; g < MAXG; ++g) {
            if (g < G) {
                const int d = __builtin_popcount(x[u] ^ st.qs[g]);
                const int t_eff = st.tt[g] + (i < st.p1[g] ? 1 : 0);   // ties before p1 are in the top m
                const bool sel = valid && (win || d < t_eff);
                const uint64_t mask = __ballot(sel);
                if (mask) {
                    const int pos = st.off[g] + (int)__builtin_amdgcn_mbcnt_hi(
                                                    (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                    if (sel && pos < a.cap) a.idx[(row0 + g) * a.cap + pos] = i;
                    st.off[g] += __popcll(mask);
                }
            }
        }
    }
}

template <int MAXG>
__global__ __launch_bounds__(64) void k_sig_compact(TopkArgs a) {
    const int lane = threadIdx.x;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int G = a.G;
    const int64_t row0 = (int64_t)b * a.Hq + h * G;
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int beg = c * kChunk;
    const int end = (int)min(a.n, (int64_t)beg + kChunk);

    uint32_t xa[16], xb[16];
    load_quarter(xa, ks, beg, end, lane);
    CompactState<MAXG> st;
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        if (g < G) {
            st.qs[g] = a.q_sigs[row0 + g];
            st.tt[g] = a.head_info[2 * (row0 + g)];
            st.p1[g] = a.head_info[2 * (row0 + g) + 1];
            st.off[g] = a.chunk_info[(row0 + g) * a.chunks + c];
        } else {
            st.qs[g] = 0;
            st.tt[g] = -1;
            st.p1[g] = 0;
            st.off[g] = 0;
        }
    }
    const int s_end = (int)min(a.n_sink, a.n), r_beg = (int)max((int64_t)0, a.n - a.n_recent);
    for (int q = 0; q < 4; q += 2) {
        const int b0 = beg + q * kQuarter, b1 = b0 + kQuarter;
        load_quarter(xb, ks, b1, end, lane);
        compact_quarter<MAXG>(a, st, xa, b0, end, row0, s_end, r_beg, lane);
        if (q + 2 < 4) load_quarter(xa, ks, b1 + kQuarter, end, lane);
        compact_quarter<MAXG>(a, st, xb, b1, end, row0, s_end, r_beg, lane);
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
        const bool sc = a.scores != nullptr;
#define LCDA_HIST(MG, V, S) hipLaunchKernelGGL((k_sig_hist<MG, V, S>), gc, dim3(64), 0, st, a)
        if (a.G <= 4) {
            if (vec) { if (sc) LCDA_HIST(4, true, true); else LCDA_HIST(4, true, false); }
            else { if (sc) LCDA_HIST(4, false, true); else LCDA_HIST(4, false, false); }
        } else {
            if (vec) { if (sc) LCDA_HIST(8, true, true); else LCDA_HIST(8, true, false); }
            else { if (sc) LCDA_HIST(8, false, true); else LCDA_HIST(8, false, false); }
        }
#undef LCDA_HIST
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_select, dim3(a.Hq, a.B), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.chunks > 0) {
        if (a.G <= 4) hipLaunchKernelGGL(k_sig_compact<4>, gc, dim3(64), 0, st, a);
        else hipLaunchKernelGGL(k_sig_compact<8>, gc, dim3(64), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace lcda
