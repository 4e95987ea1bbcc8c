// sig_topk.hip - HashAttention SCORE + TOPK over 32-bit signatures.
//
// SCORE(k_i, q) = -popcount(h_i XOR h_q) ("HashAttention: Semantic Sparsity
// for Faster Inference", slide "A 32-bit signature makes scoring cheap",
// Eq. (2)); TOPK keeps the m positions of smallest distance, ties to the lower
// position, united with the first n_sink and last n_recent positions, in
// ascending order.
//
// Distances take only 33 values, so the top m is fixed by a threshold t and a
// tie quota: every position with d < t is in, and of the positions with
// d == t the lowest `quota` are.  Split over chunks of a head's positions, the
// ties a chunk takes are its first `taken_c` ties, where taken_c follows from
// the tie counts of the chunks before it.
//
// Two kernels, each reading a KV head's codes once for all G query heads of
// its group.  The scans are bound by instruction issue
// (one xor + popcount per position and query head, plus bookkeeping), so the
// per-position work is kept to a few vector instructions.
//   1. k_topk_hist    - per chunk: the 33-bin distance histogram of each query
//                       head, in 64 per-lane LDS copies laid out so that the
//                       increments of one instruction hit distinct banks.  The
//                       last workgroup of a KV head to finish (arrival counter)
//                       then runs the selection of its G query heads:
//      select         - per query head (one wavefront, lane = chunk): t and the
//                       quota from the summed histograms, each chunk's ties
//                       taken, the window positions outside the top m in the
//                       chunks a window edge cuts (only the window part of those
//                       chunks is scanned), per-chunk output offsets, the count,
//                       the window entries of the output (its lowest and highest
//                       entries) and the -1 padding.
//   2. k_topk_compact - per chunk: each thread holds 16 consecutive positions
//                       and forms per-head 16-bit selection masks (below one
//                       threshold, plus the ties for the one chunk that takes
//                       only some of them, plus the window positions); DPP
//                       scans in each wavefront and one exchange of wavefront
//                       totals place them, and each thread stores its selected
//                       positions outside the windows.
// A chunk is a whole number of 4096-position sub-chunks, chosen so that a head
// has at most 64 chunks.  Positions are below n <= INT32_MAX; loop bounds that
// can step past n are 64-bit.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

constexpr int kSub = 4096;            // positions per sub-chunk (256 threads x 16)
constexpr int kMaxChunks = 64;        // chunks per head: one lane each in the select wavefront
constexpr int kBins = 33;
constexpr int kRow = 36;              // words per histogram row: 33 bins, padded to 9 x 16 bytes
constexpr int kPre = 8;               // window-part steps of 64 positions prefetched in the select

__device__ __forceinline__ int mbcnt64(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---- loads ------------------------------------------------------------------
// Thread tid's 16 codes of the sub-chunk at sb: positions sb + 4*(tid + 256*u) + e.
// Addresses are clamped into [.., end); entries at or past end are ignored by the caller.
template <bool VEC>
__device__ __forceinline__ void load_sub(uint32_t (&x)[16], const uint32_t* ks, int64_t sb, int64_t end, int tid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = sb + 4 * (tid + 256 * u);
        if (VEC) {
            const u32x4 v = ld16(ks + min(i, end - 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * u + e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * u + e] = ks[min(i + e, end - 1)];
        }
    }
}

// ---- selection (one wavefront per query head, lane = chunk) -------------------
// A window part [p0, p1) of a cut chunk, walked in steps of 64 positions (lane l
// of step s holds p0 + 64*s + l); the first kPre steps are requested up front.
struct Part {
    int64_t p0, p1;
    uint32_t x[kPre];
};

__device__ __forceinline__ void load_part(Part& pt, const uint32_t* ks, int lane) {
    const int64_t last = pt.p1 > pt.p0 ? pt.p1 - 1 : 0;
#pragma unroll
    for (int s = 0; s < kPre; ++s) pt.x[s] = ks[min(pt.p0 + 64 * s + lane, last)];
}

// f(i, code) for every lane's position of every step, in step order (all lanes
// call it; positions at or past p1 get some in-range code).
template <class F>
__device__ __forceinline__ void part_walk(const Part& pt, const uint32_t* ks, int lane, F&& f) {
#pragma unroll
    for (int s = 0; s < kPre; ++s)
        if (pt.p0 + 64 * s < pt.p1) f(pt.p0 + 64 * s + lane, pt.x[s]);
    for (int64_t p = pt.p0 + 64 * kPre; p < pt.p1; p += 64) f(p + lane, ks[min(p + lane, pt.p1 - 1)]);
}

// Ties (d == t) in a part.
__device__ __forceinline__ int part_ties(const Part& pt, const uint32_t* ks, uint32_t q, int t, int lane) {
    int ties = 0;
    part_walk(pt, ks, lane, [&](int64_t i, uint32_t x) {
        ties += __popcll(__ballot(i < pt.p1 && (int)__builtin_popcount(x ^ q) == t));
    });
    return ties;
}

// Positions of a part in the top m, given that tie_base ties of the chunk come
// before the part and the chunk takes its first `taken` ties.
__device__ __forceinline__ int part_top(const Part& pt, const uint32_t* ks, uint32_t q, int t, int tie_base, int taken,
                                        int lane) {
    int top = 0, carry = tie_base;
    part_walk(pt, ks, lane, [&](int64_t i, uint32_t x) {
        const int d = (int)__builtin_popcount(x ^ q);
        const bool ok = i < pt.p1;
        const uint64_t tm = __ballot(ok && d == t);
        const int rank = carry + mbcnt64(tm);
        top += __popcll(__ballot(ok && (d < t || (d == t && rank < taken))));
        carry += __popcll(tm);
    });
    return top;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ int wave_excl_scan_i(int x, int lane) {
    int inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    return inc - x;
}

__device__ void select_head(const TopkArgs& a, int b, int h, int g, int lane, uint32_t* tr /*[kBins][65]*/) {
    const int64_t row = (int64_t)b * a.Hq + h * a.G + g;
    const int64_t n = a.n;
    const int C = a.chunks;
    const int64_t len = a.chunk_len;
    const uint32_t q = a.q_sigs[row];
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * n;
    const int64_t s_end = min(a.n_sink, n);
    const int64_t r_beg = max(max((int64_t)0, n - a.n_recent), s_end);

    // Chunks cut by a window edge and the window part of each: the prefix
    // [cs*len, s_end) of the sink-cut chunk and the suffix [r_beg, end of cr) of
    // the recent-cut chunk.  Their codes do not depend on t: request them first.
    const int cs = (s_end > 0 && s_end < n && s_end % len != 0) ? (int)(s_end / len) : -1;
    const int cr = (r_beg < n && r_beg % len != 0) ? (int)(r_beg / len) : -1;
    Part ps, pr;
    ps.p0 = cs >= 0 ? cs * len : 0;
    ps.p1 = cs >= 0 ? s_end : 0;
    pr.p0 = cr >= 0 ? r_beg : 0;
    pr.p1 = cr >= 0 ? min(n, (cr + 1) * len) : 0;
    load_part(ps, ks, lane);
    load_part(pr, ks, lane);

    // This lane's chunk histogram.
    // (The other workgroups of the head wrote them: device-scope loads.)
    uint32_t hv[kBins];
    {
        const uint32_t* hrow = a.hist + (row * C + min(lane, C - 1)) * kRow;
#pragma unroll
        for (int k = 0; k < kRow / 2; ++k) {
            const uint64_t v = load_dev_u64(hrow + 2 * k);
#pragma unroll
            for (int e = 0; e < 2; ++e)
                if (2 * k + e < kBins) hv[2 * k + e] = lane < C ? (uint32_t)(v >> (32 * e)) : 0u;
        }
    }
    // The head's histogram: bins transposed through LDS, lane d (< 33) sums bin d.
#pragma unroll
    for (int d = 0; d < kBins; ++d) tr[d * 65 + lane] = hv[d];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    int64_t hsum = 0;
    if (lane < kBins) {
#pragma unroll 8
        for (int l = 0; l < 64; ++l) hsum += tr[lane * 65 + l];
    }
    // t = the first bin whose inclusive prefix reaches m; quota = what it must give (t = -1: m = 0).
    const int64_t meff = min(a.m, n);
    int64_t incl = hsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
    }
    const uint64_t reach = __ballot(lane < kBins && meff > 0 && incl >= meff);
    const int t = reach ? (int)__builtin_ctzll(reach) : -1;
    const int64_t quota = t >= 0 ? meff - (__shfl(incl, t, 64) - __shfl(hsum, t, 64)) : 0;
    int below = 0, ties = 0;
#pragma unroll
    for (int d = 0; d < kBins; ++d) {
        below += d < t ? (int)hv[d] : 0;
        ties = d == t ? (int)hv[d] : ties;
    }
    const int ties_before = wave_excl_scan_i(ties, lane);
    const int taken = t < 0 ? 0 : (int)min(max(quota - ties_before, (int64_t)0), (int64_t)ties);

    // Window positions outside the top m in the cut chunks.
    int extra_s = 0, extra_r = 0;
    if (cs >= 0) {
        const int tk = __shfl(taken, cs, 64);
        extra_s = (int)(ps.p1 - ps.p0) - part_top(ps, ks, q, t, 0, tk, lane);
    }
    if (cr >= 0) {
        const int tk = __shfl(taken, cr, 64);
        const int tie_c = __shfl(ties, cr, 64);
        const int tsuf = part_ties(pr, ks, q, t, lane);
        extra_r = (int)(pr.p1 - pr.p0) - part_top(pr, ks, q, t, tie_c - tsuf, tk, lane);
    }

    const int64_t cb = lane * len, ce = min(n, cb + len);
    int cnt = 0;
    if (lane < C) {
        if (ce <= s_end || cb >= r_beg) cnt = (int)(ce - cb);   // entirely inside a window
        else cnt = below + taken + (lane == cs ? extra_s : 0) + (lane == cr ? extra_r : 0);
    }
    const int off = wave_excl_scan_i(cnt, lane);
    const int total = wave_sum_i(cnt);
    if (lane < C) {
        // Records of one chunk for all G heads of the group sit together.
        int32_t* ci = a.chunk_info + ((((int64_t)b * a.Hkv + h) * C + lane) * a.G + g) * 4;
        ci[0] = off;
        ci[1] = taken;
        ci[2] = ties;
        ci[3] = t;
    }
    if (lane == 0) {
        a.count[row] = total;
        a.head_info[2 * row] = t;
        a.head_info[2 * row + 1] = (int32_t)quota;
    }
    // The window positions are the lowest and the highest entries of I: the
    // sink part is I[0 .. s_end) = 0 .. s_end - 1 and the recent part fills
    // the last n - r_beg entries.  They are written here; the compaction
    // counts them but stores only the positions of the top m.
    int32_t* out = a.idx + row * a.cap;
    for (int64_t i = lane; i < s_end; i += 64) out[i] = (int32_t)i;
    const int64_t nr = n - r_beg;
    for (int64_t i = lane; i < nr; i += 64) out[total - nr + i] = (int32_t)(r_beg + i);
    for (int64_t i = total + lane; i < a.cap; i += 64) out[i] = -1;
}

// ---- 1. histogram ------------------------------------------------------------------
// LDS cnt[g][bin][lane]: one copy per lane of the wavefront (the four
// wavefronts share them through atomic adds), with a spare bin 33 for
// positions past the end.  An increment's address is bin * 64 + lane, so the
// 64 lanes of one instruction fall into distinct banks whatever their bins.
template <int MAXG>
struct HistSmem {
    static constexpr int kWords = MAXG * (kBins + 1) * 64;
    uint32_t cnt[kWords];
};

// The increments of one chunk.  All MAXG heads are counted; heads at or past
// G count the codes of head G - 1 into rows that are never read, so the loop
// has no per-head branches.  FULL: the chunk is whole (every position is
// below end); otherwise positions at or past end go to the spare bin.
// The codes of kGrp sub-chunks are requested together: the ring xr holds
// them, and each slot is refilled with the sub-chunk kGrp ahead as soon as it
// has been counted, so that a group's loads are in flight at once.
constexpr int kGrp = 4;

template <bool VEC>
__device__ __forceinline__ void load_group(uint32_t (&xr)[kGrp][16], const uint32_t* ks, int64_t gb, int64_t end,
                                           int tid) {
#pragma unroll
    for (int u = 0; u < kGrp; ++u)
        if (gb + (int64_t)u * kSub < end) load_sub<VEC>(xr[u], ks, gb + (int64_t)u * kSub, end, tid);
}

template <int MAXG, bool VEC, bool FULL, bool SCORES>
__device__ __forceinline__ void hist_chunk(const TopkArgs& a, uint32_t* my, const uint32_t* ks,
                                           const uint32_t (&qs)[MAXG], uint32_t (&xr)[kGrp][16], int64_t beg,
                                           int64_t end, int tid, int64_t row0) {
    for (int64_t gb = beg; gb < end; gb += (int64_t)kGrp * kSub) {
#pragma unroll
        for (int u = 0; u < kGrp; ++u) {
            const int64_t sb = gb + (int64_t)u * kSub;
            if (sb < end) {   // uniform
                uint32_t x[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) x[k] = xr[u][k];
                const int64_t nb = sb + (int64_t)kGrp * kSub;
                if (nb < end) load_sub<VEC>(xr[u], ks, nb, end, tid);
                const int rem = FULL ? kSub : (int)min(end - sb, (int64_t)kSub);
#pragma unroll
                for (int uu = 0; uu < 4; ++uu) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int k = 4 * (tid + 256 * uu) + e;
                        const bool ok = FULL || k < rem;
#pragma unroll
                        for (int g = 0; g < MAXG; ++g) {
                            const uint32_t d = __builtin_popcount(x[4 * uu + e] ^ qs[g]);
                            const uint32_t bin = ok ? d : (uint32_t)kBins;
                            uint32_t* p = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(my) + (bin << 8)) +
                                          g * (kBins + 1) * 64;
                            __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                            if (SCORES && ok && g < a.G)
                                a.scores[(row0 + g) * a.n + sb + k] = (int8_t)(-(int)d);
                        }
                    }
                }
            }
        }
    }
}

template <int MAXG, bool VEC, bool SCORES>
__global__ __launch_bounds__(256) void k_topk_hist(TopkArgs a) {
    __shared__ HistSmem<MAXG> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int G = a.G;
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int64_t beg = (int64_t)c * a.chunk_len;
    const int64_t end = min(a.n, beg + a.chunk_len);
    const int64_t row0 = (int64_t)b * a.Hq + h * G;

    uint32_t xr[kGrp][16];
    load_group<VEC>(xr, ks, beg, end, tid);
    static_assert(HistSmem<MAXG>::kWords % 4 == 0, "zeroed in 16-byte stores");
    for (int k = 4 * tid; k < HistSmem<MAXG>::kWords; k += 4 * 256)
        *reinterpret_cast<u32x4*>(sm.cnt + k) = u32x4{0u, 0u, 0u, 0u};
    uint32_t qs[MAXG];
#pragma unroll
    for (int g = 0; g < MAXG; ++g) qs[g] = a.q_sigs[row0 + min(g, G - 1)];
    __syncthreads();

    uint32_t* my = sm.cnt + lane;
    if (end - beg == a.chunk_len) hist_chunk<MAXG, VEC, true, SCORES>(a, my, ks, qs, xr, beg, end, tid, row0);
    else hist_chunk<MAXG, VEC, false, SCORES>(a, my, ks, qs, xr, beg, end, tid, row0);
    __syncthreads();
    // Sum the 64 copies of each (head, bin); each thread starts at its own
    // lane copy so that the reads of one instruction fall into distinct banks.
    for (int k = tid; k < G * kBins; k += 256) {
        const int g = k / kBins, bin = k % kBins;
        const uint32_t* row = sm.cnt + (g * (kBins + 1) + bin) * 64;
        uint32_t sum = 0;
#pragma unroll 8
        for (int l = 0; l < 64; ++l) sum += row[(l + tid) & 63];
        store_dev(a.hist + (((int64_t)b * a.Hq + h * G + g) * a.chunks + c) * kRow + bin, sum);
    }

    // The head's last workgroup to finish selects for its G query heads (one
    // wavefront each), reusing the counters' LDS.
    __shared__ int s_last;
    if (arrive_count(a.ctr + (int64_t)b * a.Hkv + h, (uint32_t)a.chunks, &s_last)) {
        uint32_t* tr = sm.cnt + (tid >> 6) * (kBins * 65);
        static_assert(4 * kBins * 65 <= HistSmem<MAXG>::kWords, "select scratch fits the counters' LDS");
        for (int g = tid >> 6; g < G; g += 4) select_head(a, b, h, g, lane, tr);
    }
}

// n == 0: no positions; every row gets count 0 and is padded with -1.
__global__ __launch_bounds__(64) void k_topk_empty(TopkArgs a) {
    const int64_t row = (int64_t)blockIdx.y * a.Hq + blockIdx.x;
    if (threadIdx.x == 0) a.count[row] = 0;
    for (int64_t i = threadIdx.x; i < a.cap; i += 64) a.idx[row * a.cap + i] = -1;
}

// ---- 3. ordered compaction -------------------------------------------------------
// Thread tid owns the 16 consecutive positions sb + 16*tid + j of a sub-chunk.
// Per query head it forms a 16-bit selection mask; the exclusive prefix of the
// masks' popcounts over the threads (two heads packed in the 16-bit fields of
// a word) places every thread's positions, which it then stores in order.
// The prefix is a DPP scan inside each wavefront plus the wavefront totals
// exchanged through LDS.  A head that takes only some of the chunk's ties
// first needs the ties before each thread: the same scan over the tie counts,
// run only when some head does.
template <bool VEC>
__device__ __forceinline__ void load_run(uint32_t (&x)[16], const uint32_t* ks, int64_t sb, int64_t end, int tid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = sb + 16 * tid + 4 * u;
        if (VEC) {
            const u32x4 v = ld16(ks + min(i, end - 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * u + e] = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * u + e] = ks[min(i + e, end - 1)];
        }
    }
}

// Inclusive scan over the 64 lanes of a wavefront: sums within rows of 16 by
// shifts of 1, 2, 4 and 8 lanes (zero filled at the row start), then the last
// lane of row 0 (of row 2) is added to row 1 (row 3), and the last lane of
// row 1 to rows 2 and 3.  Words hold two 16-bit counts that never carry.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return x;
}

__device__ __forceinline__ int field16(uint32_t v, int k) { return (int)((v >> (16 * k)) & 0xFFFFu); }

// The lowest `take` set bits of m.
__device__ __forceinline__ uint32_t lowest_bits(uint32_t m, int take) {
    uint32_t r = 0;
    for (int j = 0; j < take && m; ++j) {
        const uint32_t low = m & (0u - m);
        r |= low;
        m ^= low;
    }
    return r;
}

// Bit j of the result: position j of the thread's 16 has popcount(code ^ q) <
// thr.  The bits are shifted in from the top position down, each as the sign
// of popcount + nthr (nthr = -thr, kept opaque so that the add folds into the
// popcount), funnelled in by one alignbit.
__device__ __forceinline__ uint32_t below_mask(const uint32_t (&x)[16], uint32_t q, uint32_t nthr) {
    uint32_t m = 0;
#pragma unroll
    for (int j = 15; j >= 0; --j)
        m = __builtin_amdgcn_alignbit(m, (uint32_t)__builtin_popcount(x[j] ^ q) + nthr, 31);
    return m;
}

// Window positions among the thread's 16 positions i0 .. i0 + 15: below s_end
// or at / past r_beg.
__device__ __forceinline__ uint32_t window_mask(int64_t i0, int64_t s_end, int64_t r_beg) {
    const int lo = (int)min(max(s_end - i0, (int64_t)0), (int64_t)16);   // positions below s_end
    const int hi = (int)min(max(r_beg - i0, (int64_t)0), (int64_t)16);   // positions below r_beg
    const uint32_t below_s = lo >= 16 ? 0xFFFFu : ((1u << lo) - 1u);
    const uint32_t from_r = hi >= 16 ? 0u : (0xFFFFu & ~((1u << hi) - 1u));
    return below_s | from_r;
}

// Sub-chunks are handled in groups of kGrp: the masks and in-wavefront scans
// of the whole group first, then one exchange of the wavefront totals (one
// barrier; a second one for the tie ranks of a head taking only some of the
// chunk's ties), then the stores.  The codes come through a ring of kGrp
// sub-chunks, as in the histogram.
template <bool VEC>
__device__ __forceinline__ void load_run_group(uint32_t (&xr)[kGrp][16], const uint32_t* ks, int64_t gb, int64_t end,
                                               int tid) {
#pragma unroll
    for (int u = 0; u < kGrp; ++u)
        if (gb + (int64_t)u * kSub < end) load_run<VEC>(xr[u], ks, gb + (int64_t)u * kSub, end, tid);
}

template <int MAXG, bool VEC>
__global__ __launch_bounds__(256) void k_topk_compact(TopkArgs a) {
    constexpr int kW = MAXG / 2;                 // words of packed 16-bit counts
    __shared__ uint32_t sh[2][2][kGrp][4][kW];   // [parity][selection, ties][sub][wavefront][word]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int G = a.G;
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int64_t beg = (int64_t)c * a.chunk_len;
    const int64_t end = min(a.n, beg + a.chunk_len);
    const int64_t s_end = min(a.n_sink, a.n);
    const int64_t r_beg = max((int64_t)0, a.n - a.n_recent);
    const bool meets_win = beg < s_end || end > r_beg;   // uniform
    const int64_t row0 = (int64_t)b * a.Hq + h * G;

    uint32_t xr[kGrp][16];
    load_run_group<VEC>(xr, ks, beg, end, tid);
    // The chunk's records of all heads, {off, taken, ties, t} each, in one block.
    // Per head: the selection below threshold thr (t, or t + 1 for a chunk that
    // takes all its ties); a chunk that takes only some of its ties (mode 2)
    // also forms the tie mask.  Heads at or past G select nothing.
    const int32_t* rec = a.chunk_info + (((int64_t)b * a.Hkv + h) * a.chunks + c) * G * 4;
    uint32_t q[MAXG], nthr[MAXG], nt1[MAXG];
    int off[MAXG], taken[MAXG], mode[MAXG], tie_carry[MAXG];   // mode: 0 no ties, 1 all ties, 2 some ties
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        const int gg = min(g, G - 1);
        const int32_t* ci = rec + 4 * gg;
        q[g] = a.q_sigs[row0 + gg];
        const int t = g < G ? ci[3] : -1;
        off[g] = ci[0];
        taken[g] = ci[1];
        const int ties = ci[2];
        mode[g] = (t < 0 || taken[g] == 0) ? 0 : (taken[g] == ties ? 1 : 2);
        nthr[g] = (uint32_t)__builtin_amdgcn_readfirstlane(-(t + (mode[g] == 1 ? 1 : 0)));
        nt1[g] = (uint32_t)__builtin_amdgcn_readfirstlane(-(t + 1));
        tie_carry[g] = 0;
    }
    bool partial = false;   // uniform: every thread read the same chunk records
#pragma unroll
    for (int g = 0; g < MAXG; ++g) partial |= mode[g] == 2;
    // Rows whose byte offsets fit 32 bits are stored through a buffer
    // resource (offset arithmetic in 32 bits, the range check in hardware).
    const bool small_cap = a.cap < ((int64_t)1 << 29);

    int par = 0;
    for (int64_t gb = beg; gb < end; gb += (int64_t)kGrp * kSub, par ^= 1) {
        // Selection masks (two heads per word, 16 bits each) and their counts.
        uint32_t sel[kGrp][kW], cnt[kGrp][kW], inc[kGrp][kW];
        uint32_t tie[kGrp][kW], tcnt[kGrp][kW], tinc[kGrp][kW];
#pragma unroll
        for (int u = 0; u < kGrp; ++u) {
            const int64_t sb = gb + (int64_t)u * kSub;
            uint32_t x[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) x[k] = xr[u][k];
            if (sb + (int64_t)kGrp * kSub < end) load_run<VEC>(xr[u], ks, sb + (int64_t)kGrp * kSub, end, tid);
            const int64_t i0 = sb + 16 * tid;
            const int nv = (int)max((int64_t)0, min((int64_t)16, end - i0));   // valid positions of this thread
            const uint32_t valid = nv >= 16 ? 0xFFFFu : ((1u << nv) - 1u);
            const uint32_t win = meets_win ? window_mask(i0, s_end, r_beg) & valid : 0u;
#pragma unroll
            for (int k = 0; k < kW; ++k) {
                uint32_t m2[2], t2[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int g = 2 * k + e;
                    uint32_t sm, tm = 0;
                    if (partial && mode[g] == 2) {   // uniform
                        // d < t and d <= t from the same popcounts; ties rank over every
                        // position of the chunk, window positions included.
                        uint32_t l = 0, le = 0;
#pragma unroll
                        for (int jj = 15; jj >= 0; --jj) {
                            const uint32_t pc = (uint32_t)__builtin_popcount(x[jj] ^ q[g]);
                            l = __builtin_amdgcn_alignbit(l, pc + nthr[g], 31);
                            le = __builtin_amdgcn_alignbit(le, pc + nt1[g], 31);
                        }
                        sm = l & valid;
                        tm = le & ~l & valid;
                    } else {
                        sm = below_mask(x, q[g], nthr[g]) & valid;
                    }
                    m2[e] = g < G ? (sm | win) : 0u;
                    t2[e] = tm;
                }
                sel[u][k] = m2[0] | (m2[1] << 16);
                tie[u][k] = t2[0] | (t2[1] << 16);
                tcnt[u][k] = (uint32_t)__builtin_popcount(t2[0]) | ((uint32_t)__builtin_popcount(t2[1]) << 16);
                tinc[u][k] = partial ? wave_incl_scan(tcnt[u][k]) : 0u;
                if (partial && lane == 63) sh[par][1][u][w][k] = tinc[u][k];
            }
        }
        if (partial) {
            // Tie ranks: a head taking only some of the chunk's ties takes the
            // lowest `taken - ties before` ties of each thread.
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kW; ++k) {
                uint32_t run = 0;   // ties of the sub-chunks before, in this group
#pragma unroll
                for (int u = 0; u < kGrp; ++u) {
                    uint32_t base = 0, all = 0;
#pragma unroll
                    for (int ww = 0; ww < 4; ++ww) {
                        const uint32_t tw = sh[par][1][u][ww][k];
                        base += ww < w ? tw : 0u;
                        all += tw;
                    }
                    const uint32_t before2 = run + base + tinc[u][k] - tcnt[u][k];
                    run += all;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int g = 2 * k + e;
                        if (mode[g] == 2) {
                            const int before = tie_carry[g] + field16(before2, e);
                            const uint32_t tk =
                                lowest_bits((tie[u][k] >> (16 * e)) & 0xFFFFu, min(max(taken[g] - before, 0), 16));
                            sel[u][k] |= tk << (16 * e);
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 2; ++e) tie_carry[2 * k + e] += field16(run, e);
            }
        }
#pragma unroll
        for (int u = 0; u < kGrp; ++u) {
#pragma unroll
            for (int k = 0; k < kW; ++k) {
                cnt[u][k] = (uint32_t)__builtin_popcount(sel[u][k] & 0xFFFFu) |
                            ((uint32_t)__builtin_popcount(sel[u][k] >> 16) << 16);
                inc[u][k] = wave_incl_scan(cnt[u][k]);
                if (lane == 63) sh[par][0][u][w][k] = inc[u][k];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kW; ++k) {
            uint32_t run = 0;   // selected positions of the sub-chunks before, in this group
#pragma unroll
            for (int u = 0; u < kGrp; ++u) {
                uint32_t base = 0, all = 0;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) {
                    const uint32_t sw = sh[par][0][u][ww][k];
                    base += ww < w ? sw : 0u;
                    all += sw;
                }
                const uint32_t ex2 = run + base + inc[u][k] - cnt[u][k];
                run += all;
                const int64_t i0 = gb + (int64_t)u * kSub + 16 * tid;
                // Window positions were stored by the select: skip them, keeping
                // the ranks of the others.  The buffer resource bounds every
                // store to the row (cap entries).
                const uint32_t win = meets_win ? window_mask(i0, s_end, r_beg) : 0u;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int g = 2 * k + e;
                    if (g < G) {
                        const uint32_t mine = (sel[u][k] >> (16 * e)) & 0xFFFFu;
                        const uint32_t wm = mine & win;   // window positions among them
                        uint32_t m = mine ^ wm;
                        if (__ballot(m != 0u)) {
                            const int base = off[g] + field16(ex2, e);
                            int32_t* out = a.idx + (row0 + g) * a.cap;
                            if (small_cap) {
                                const __amdgpu_buffer_rsrc_t ro =
                                    __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)(a.cap * 4), kRsrcWord3);
                                uint32_t pos4 = 4u * (uint32_t)base;
                                if (__ballot(wm != 0u)) {
                                    // a kept position's slot also counts the window positions before it
                                    while (m) {
                                        const int j = __builtin_ctz(m);
                                        const uint32_t w4 = 4u * (uint32_t)__builtin_popcount(wm & ((1u << j) - 1u));
                                        __builtin_amdgcn_raw_buffer_store_b32((int)(i0 + j), ro, pos4 + w4, 0, 0);
                                        pos4 += 4u;
                                        m &= m - 1u;
                                    }
                                } else {
                                    while (m) {
                                        const int j = __builtin_ctz(m);
                                        __builtin_amdgcn_raw_buffer_store_b32((int)(i0 + j), ro, pos4, 0, 0);
                                        pos4 += 4u;
                                        m &= m - 1u;
                                    }
                                }
                            } else {
                                while (m) {
                                    const int j = __builtin_ctz(m);
                                    const int pos = base + __builtin_popcount(mine & ((1u << j) - 1u));
                                    if (pos < a.cap) out[pos] = (int32_t)(i0 + j);
                                    m &= m - 1u;
                                }
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) off[2 * k + e] += field16(run, e);
        }
    }
}

}  // namespace

int topk_chunk_len(int64_t n) {
    const int64_t per = (int64_t)kSub * kMaxChunks;
    const int64_t subs = n > 0 ? (n + per - 1) / per : 1;
    return (int)(max(subs, tuning().topk_subs) * kSub);
}

int topk_hist_row() { return kRow; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    if (a.B <= 0) return hipSuccess;
    if (a.G > 8 || a.chunks > kMaxChunks) return hipErrorInvalidValue;
    if (a.chunks == 0) {
        hipLaunchKernelGGL(k_topk_empty, dim3(a.Hq, a.B), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    const dim3 grid(a.chunks, a.Hkv, a.B), block(256);
    const bool vec = a.n % 4 == 0;
    const bool sc = a.scores != nullptr;
#define LCDA_HIST(MG, V, S) hipLaunchKernelGGL((k_topk_hist<MG, V, S>), grid, block, 0, st, a)
    if (a.G <= 4) {
        if (vec) { if (sc) LCDA_HIST(4, true, true); else LCDA_HIST(4, true, false); }
        else { if (sc) LCDA_HIST(4, false, true); else LCDA_HIST(4, false, false); }
    } else {
        if (vec) { if (sc) LCDA_HIST(8, true, true); else LCDA_HIST(8, true, false); }
        else { if (sc) LCDA_HIST(8, false, true); else LCDA_HIST(8, false, false); }
    }
#undef LCDA_HIST
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.G <= 4) {
        if (vec) hipLaunchKernelGGL((k_topk_compact<4, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_topk_compact<4, false>), grid, block, 0, st, a);
    } else {
        if (vec) hipLaunchKernelGGL((k_topk_compact<8, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_topk_compact<8, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace lcda
