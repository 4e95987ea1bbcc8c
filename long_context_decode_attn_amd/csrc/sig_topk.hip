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
//                       increments of one instruction hit distinct banks.  A
//                       chunk that a window edge cuts also histograms its
//                       window part.
//   2. k_topk_compact - per chunk, first the selection: per query head (one
//                       wavefront, lane = chunk), t and the quota from the
//                       summed histograms, each chunk's ties taken, the window
//                       positions outside the top m (from the window parts'
//                       histograms) and the chunks' output offsets; every
//                       workgroup of a head computes them while its codes are
//                       on their way, and the one of chunk 0 writes the count,
//                       the window entries of the output (its lowest and highest
//                       entries) and the -1 padding.  Then each thread holds 16
//                       consecutive positions and forms per-head 16-bit
//                       selection masks (below one threshold, plus the ties for
//                       the one chunk that takes only some of them, plus the
//                       window positions); DPP scans in each wavefront and one
//                       exchange of wavefront totals place them, and each thread
//                       stores its selected positions outside the windows.
// A chunk is a whole number of 4096-position sub-chunks, chosen so that a head
// has at most 64 chunks.  Positions are below n <= INT32_MAX; loop bounds that
// can step past n are 64-bit.

#include "common.h"
#include "internal.h"
#include "sparse.h"
#include "sig_proj.h"

namespace lcda {
namespace {

constexpr int kSub = 4096;            // positions per sub-chunk (256 threads x 16)
constexpr int kMaxChunks = 64;        // chunks per head: one lane each in the select wavefront
constexpr int kBins = 33;
constexpr int kRow = 36;              // words per histogram row: 33 bins, padded to 9 x 16 bytes
constexpr int kTr = 68;               // words per bin in the selection's transposition: 64 chunks + 4

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

// ---- 0. query codes at the head of the histogram pass ----------------------------
// R ([128][32], columns at or past `bits` zero, so those bits come out 0) and
// the G query rows (as floats) are staged in LDS with one round of loads, so
// that the chains wait on memory once.  Thread t < 32 * G computes bit t % 32
// of head t / 32's code, and each wavefront's ballot packs two heads' codes.
__device__ void encode_q_heads(const TopkArgs& a, int64_t row0, int tid, float* sR /* [128 * 32 + 8 * 128] */,
                               uint32_t* s_codes /* [8] */) {
    float* sQ = sR + kD * 32;
    for (int k = tid; k < kD * 32; k += 256) {
        const int e = k >> 5, b = k & 31;
        sR[k] = b < a.bits ? a.R[e * a.bits + b] : 0.f;
    }
    for (int k = tid; k < a.G * kD; k += 256) {
        const int64_t i = row0 * kD + k;
        sQ[k] = a.q_bf16 ? bf16_lo(static_cast<const uint16_t*>(a.q)[i]) : static_cast<const float*>(a.q)[i];
    }
    __syncthreads();
    const int g = min(tid >> 5, a.G - 1), b = tid & 31;
    const float* xr = sQ + g * kD;
    const double z = proj_chain([&](int e) { return xr[e]; }, sR + b, 32);
    const uint64_t bits = __ballot(z > 0.0);
    const int h0 = 2 * (tid >> 6);
    if ((tid & 63) == 0 && h0 < a.G) s_codes[h0] = (uint32_t)bits;
    if ((tid & 63) == 32 && h0 + 1 < a.G) s_codes[h0 + 1] = (uint32_t)(bits >> 32);
}

// ---- 1. histogram ------------------------------------------------------------------
// LDS cnt[g][bin][lane]: one copy per lane of the wavefront (the four
// wavefronts share them through atomic adds), with a spare bin 33 for
// positions past the end.  An increment's address is bin * 64 + lane, so the
// 64 lanes of one instruction fall into distinct banks whatever their bins.
template <int MAXG>
struct __align__(16) HistSmem {
    static constexpr int kWords = MAXG * (kBins + 1) * 64;
    static constexpr int kPartWords = 2 * MAXG * kBins;
    uint32_t cnt[kWords];
    uint32_t part[kPartWords];   // [sink part, recent part][head][bin], shared by all lanes
};

// The increments of one chunk.  All MAXG heads are counted; heads at or past
// G count the codes of head G - 1 into rows that are never read, so the loop
// has no per-head branches.  FULL: the chunk is whole (every position is
// below end); otherwise positions at or past end go to the spare bin.
// The codes of kGrp sub-chunks are requested together: the ring xr holds
// them, and each slot is refilled with the sub-chunk kGrp ahead as soon as it
// has been counted, so that a group's loads are in flight at once.
constexpr int kGrp = 4;

template <bool VEC, int NG>
__device__ __forceinline__ void load_group(uint32_t (&xr)[NG][16], const uint32_t* ks, int64_t gb, int64_t end,
                                           int tid) {
#pragma unroll
    for (int u = 0; u < NG; ++u)
        if (gb + (int64_t)u * kSub < end) load_sub<VEC>(xr[u], ks, gb + (int64_t)u * kSub, end, tid);
}

// The window parts of a chunk that a window edge cuts are counted as well,
// into counters that all lanes share: positions below s_cut (the sink part;
// s_cut = beg when the chunk is not cut there) and from r_cut (the recent part;
// r_cut = end when not cut).  Only the sub-chunks that meet a part do this.
template <int MAXG, bool VEC, bool FULL, bool SCORES, int NG>
__device__ __forceinline__ void hist_chunk(const TopkArgs& a, uint32_t* my, uint32_t* part, const uint32_t* ks,
                                           const uint32_t (&qs)[MAXG], uint32_t (&xr)[NG][16], int64_t beg,
                                           int64_t end, int64_t s_cut, int64_t r_cut, int tid, int64_t row0) {
    for (int64_t gb = beg; gb < end; gb += (int64_t)NG * kSub) {
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int64_t sb = gb + (int64_t)u * kSub;
            if (sb < end) {   // uniform
                uint32_t x[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) x[k] = xr[u][k];
                const int64_t nb = sb + (int64_t)NG * kSub;
                if (nb < end) load_sub<VEC>(xr[u], ks, nb, end, tid);
                const int rem = FULL ? kSub : (int)min(end - sb, (int64_t)kSub);
                if (sb < s_cut || min(sb + (int64_t)kSub, end) > r_cut) {   // uniform
                    // Offsets from sb: the sink part is below s_rel, the recent part in [r_rel, rem).
                    const int s_rel = (int)max(min(s_cut - sb, (int64_t)kSub), (int64_t)0);
                    const int r_rel = (int)max(min(r_cut - sb, (int64_t)kSub), (int64_t)0);
#pragma unroll
                    for (int uu = 0; uu < 4; ++uu) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int k = 4 * (tid + 256 * uu) + e;
                            const int pt = k < s_rel ? 0 : (k >= r_rel && k < rem ? 1 : -1);
                            if (pt >= 0) {
#pragma unroll
                                for (int g = 0; g < MAXG; ++g)
                                    __hip_atomic_fetch_add(part + (pt * MAXG + g) * kBins +
                                                               __builtin_popcount(x[4 * uu + e] ^ qs[g]),
                                                           1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                            }
                        }
                    }
                }
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

template <int MAXG>
__device__ __forceinline__ void zero_counters(HistSmem<MAXG>& sm, int tid) {
    static_assert(HistSmem<MAXG>::kWords % 4 == 0, "zeroed in 16-byte stores");
    for (int k = 4 * tid; k < HistSmem<MAXG>::kWords; k += 4 * 256)
        *reinterpret_cast<u32x4*>(sm.cnt + k) = u32x4{0u, 0u, 0u, 0u};
    for (int k = tid; k < HistSmem<MAXG>::kPartWords; k += 256) sm.part[k] = 0u;
}

// Sum the 64 copies of each (head, bin) into histogram row `slot` of each of
// the G heads; each thread starts at its own lane copy so that the reads of
// one instruction fall into distinct banks.
template <int MAXG>
__device__ __forceinline__ void store_rows(const HistSmem<MAXG>& sm, const TopkArgs& a, int64_t row0, int slot,
                                           int tid) {
    for (int k = tid; k < a.G * kBins; k += 256) {
        const int g = k / kBins, bin = k % kBins;
        const uint32_t* r = sm.cnt + (g * (kBins + 1) + bin) * 64;
        uint32_t sum = 0;
#pragma unroll 8
        for (int l = 0; l < 64; ++l) sum += r[(l + tid) & 63];
        a.hist[((row0 + g) * (a.chunks + 2) + slot) * kRow + bin] = sum;
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

    // With the score stores and four heads, a ring of four sub-chunks went to scratch memory; two stay in
    // registers (the compiler keeps the ring of four in registers for eight heads).
    constexpr int NG = (SCORES && MAXG == 4) ? 2 : kGrp;
    uint32_t xr[NG][16];
    load_group<VEC>(xr, ks, beg, end, tid);
    uint32_t qs[MAXG];
    __shared__ uint32_t s_qc[8];
    if (a.q != nullptr) {   // uniform: the query codes are encoded here (T_map), while the codes load
        static_assert(HistSmem<MAXG>::kWords >= kD * 32 + 8 * kD, "R and the query rows fit the counters' LDS");
        encode_q_heads(a, row0, tid, reinterpret_cast<float*>(sm.cnt), s_qc);   // before the counters are zeroed
        __syncthreads();
#pragma unroll
        for (int g = 0; g < MAXG; ++g) qs[g] = s_qc[min(g, G - 1)];
        if (c == 0 && tid < G) a.q_codes[row0 + tid] = s_qc[tid];   // for the compaction
    } else {
#pragma unroll
        for (int g = 0; g < MAXG; ++g) qs[g] = a.q_sigs[row0 + min(g, G - 1)];
    }
    zero_counters(sm, tid);
    __syncthreads();

    // A chunk that a window edge cuts also counts its window part (the prefix
    // below s_end, the suffix from r_beg) into rows chunks and chunks + 1.
    const int64_t s_end = min(a.n_sink, a.n);
    const int64_t r_beg = max(max((int64_t)0, a.n - a.n_recent), s_end);
    const int64_t s_cut = (beg < s_end && s_end < end) ? s_end : beg;
    const int64_t r_cut = (beg < r_beg && r_beg < end) ? r_beg : end;
    uint32_t* my = sm.cnt + lane;
    if (end - beg == a.chunk_len)
        hist_chunk<MAXG, VEC, true, SCORES, NG>(a, my, sm.part, ks, qs, xr, beg, end, s_cut, r_cut, tid, row0);
    else
        hist_chunk<MAXG, VEC, false, SCORES, NG>(a, my, sm.part, ks, qs, xr, beg, end, s_cut, r_cut, tid, row0);
    __syncthreads();
    store_rows(sm, a, row0, c, tid);

    for (int k = tid; k < 2 * a.G * kBins; k += 256) {
        const int pt = k / (a.G * kBins), g = (k / kBins) % a.G, bin = k % kBins;
        if (pt == 0 ? s_cut > beg : r_cut < end)
            a.hist[((row0 + g) * (a.chunks + 2) + a.chunks + pt) * kRow + bin] = sm.part[(pt * MAXG + g) * kBins + bin];
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

// ---- 2. selection (in every compaction workgroup) -----------------------------------
// One wavefront per query head, lane = chunk, from the histograms of all the
// head's chunks: t and the quota, the ties each chunk takes (the ties of the
// chunks before it come first), the window positions outside the top m in the
// chunks a window edge cuts (from the histograms of their window parts), and
// each chunk's output offset.  Every compaction workgroup of a head computes
// the same values and keeps its own chunk's; the workgroup of chunk 0 also
// writes the count, the window entries of the output (its lowest and highest
// entries) and the -1 padding.
struct ChunkRec {
    int off, taken, ties, t;
};

__device__ __forceinline__ uint32_t lane_of(uint32_t x, int l) {   // l uniform
    return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

// The histograms one selection reads: this lane's chunk histogram, and bin
// `lane` of the two window parts (zero where no chunk is cut).
struct SelIn {
    uint32_t hv[kRow];
    uint32_t ps, pr;
};

__device__ __forceinline__ void window_cuts(const TopkArgs& a, int64_t& s_end, int64_t& r_beg, int& cs, int& cr) {
    s_end = min(a.n_sink, a.n);
    r_beg = max(max((int64_t)0, a.n - a.n_recent), s_end);
    cs = (s_end > 0 && s_end < a.n && s_end % a.chunk_len != 0) ? (int)(s_end / a.chunk_len) : -1;   // sink-cut chunk
    cr = (r_beg < a.n && r_beg % a.chunk_len != 0) ? (int)(r_beg / a.chunk_len) : -1;               // recent-cut chunk
}

__device__ __forceinline__ void select_load(const TopkArgs& a, int64_t row, int lane, SelIn& in) {
    int64_t s_end, r_beg;
    int cs, cr;
    window_cuts(a, s_end, r_beg, cs, cr);
    const int C = a.chunks;
    const uint32_t* hrow = a.hist + row * (C + 2) * kRow;
#pragma unroll
    for (int k = 0; k < kRow / 4; ++k) {
        const u32x4 v = lane < C ? *reinterpret_cast<const u32x4*>(hrow + lane * kRow + 4 * k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) in.hv[4 * k + e] = v[e];
    }
    in.ps = (cs >= 0 && lane < kBins) ? hrow[C * kRow + lane] : 0u;
    in.pr = (cr >= 0 && lane < kBins) ? hrow[(C + 1) * kRow + lane] : 0u;
}

__device__ ChunkRec select_chunk(const TopkArgs& a, int64_t row, int c, int lane, const SelIn& in,
                                 uint32_t* tr /*[kBins][kTr]*/) {
    const int64_t n = a.n;
    const int C = a.chunks;
    const int64_t len = a.chunk_len;
    int64_t s_end, r_beg;
    int cs, cr;
    window_cuts(a, s_end, r_beg, cs, cr);
    const uint32_t* hv = in.hv;
    const uint32_t ps = in.ps, pr = in.pr;

    // The head's histogram: bins transposed through LDS, lane d (< 33) sums bin d.
#pragma unroll
    for (int d = 0; d < kBins; ++d) tr[d * kTr + lane] = hv[d];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint32_t hsum = 0;
    if (lane < kBins) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(tr + lane * kTr + 4 * k);
            hsum += (v[0] + v[1]) + (v[2] + v[3]);
        }
    }
    // t = the first bin whose inclusive prefix reaches m; quota = what it must
    // give (t = -1: m = 0).  Counts stay below n <= INT32_MAX.
    const uint32_t meff = (uint32_t)min(a.m, n);
    const uint32_t incl = wave_incl_scan(hsum);
    const uint64_t reach = __ballot(lane < kBins && meff > 0 && incl >= meff);
    const int t = reach ? (int)__builtin_ctzll(reach) : -1;
    const int tl = t >= 0 ? t : 0;
    const int quota = t >= 0 ? (int)(meff - (lane_of(incl, tl) - lane_of(hsum, tl))) : 0;
    uint32_t below = 0, ties = 0;
#pragma unroll
    for (int d = 0; d < kBins; ++d) {
        below += d < t ? hv[d] : 0u;
        ties = d == t ? hv[d] : ties;
    }
    const int ties_before = (int)(wave_incl_scan(ties) - ties);
    const int taken = t < 0 ? 0 : min(max(quota - ties_before, 0), (int)ties);

    // Window positions outside the top m in the cut chunks.  The ties a chunk
    // takes are its first ones: the sink part (a prefix) takes the first of
    // them, the recent part (a suffix) what is left after the ties before it.
    int extra_s = 0, extra_r = 0;
    if (cs >= 0) {
        int top = 0;
        if (t >= 0)
            top = (int)(lane_of(wave_incl_scan(lane < t ? ps : 0u), 63)) +
                  min((int)lane_of(ps, tl), (int)lane_of((uint32_t)taken, cs));
        extra_s = (int)(s_end - (int64_t)cs * len) - top;
    }
    if (cr >= 0) {
        int top = 0;
        if (t >= 0) {
            const int tp = (int)lane_of(pr, tl);
            const int before = (int)lane_of(ties, cr) - tp;
            top = (int)(lane_of(wave_incl_scan(lane < t ? pr : 0u), 63)) +
                  min(max((int)lane_of((uint32_t)taken, cr) - before, 0), tp);
        }
        extra_r = (int)(min(n, (int64_t)(cr + 1) * len) - r_beg) - top;
    }

    const int64_t cb = (int64_t)lane * len, ce = min(n, cb + len);
    uint32_t cnt = 0;
    if (lane < C) {
        if (ce <= s_end || cb >= r_beg) cnt = (uint32_t)(ce - cb);   // entirely inside a window
        else cnt = below + (uint32_t)taken + (uint32_t)(lane == cs ? extra_s : 0) + (uint32_t)(lane == cr ? extra_r : 0);
    }
    const uint32_t cincl = wave_incl_scan(cnt);
    const int total = (int)lane_of(cincl, 63);

    if (c == 0) {   // uniform
        if (lane == 0) a.count[row] = total;
        // The window positions are the lowest and the highest entries of I:
        // the sink part is I[0 .. s_end) = 0 .. s_end - 1 and the recent part
        // fills the last n - r_beg entries.  The compaction stores only the
        // positions of the top m.
        int32_t* out = a.idx + row * a.cap;
        for (int64_t i = lane; i < s_end; i += 64) out[i] = (int32_t)i;
        const int64_t nr = n - r_beg;
        for (int64_t i = lane; i < nr; i += 64) out[total - nr + i] = (int32_t)(r_beg + i);
        for (int64_t i = total + lane; i < a.cap; i += 64) out[i] = -1;
    }
    return ChunkRec{(int)(lane_of(cincl, c) - lane_of(cnt, c)), (int)lane_of((uint32_t)taken, c),
                    (int)lane_of(ties, c), t};
}

template <int MAXG, bool VEC>
__global__ __launch_bounds__(256) void k_topk_compact(TopkArgs a) {
    constexpr int kW = MAXG / 2;                 // words of packed 16-bit counts
    __shared__ uint32_t sh[2][2][kGrp][4][kW];   // [parity][selection, ties][sub][wavefront][word]
    __shared__ __align__(16) uint32_t s_tr[4][kBins * kTr];   // the selection's transposition, one per wavefront
    __shared__ int s_rec[MAXG][4];
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

    // The chunk's records of all heads, {off, taken, ties, t} each, while the
    // codes are on their way.  Per head: the selection below threshold thr (t,
    // or t + 1 for a chunk that takes all its ties); a chunk that takes only
    // some of its ties (mode 2) also forms the tie mask.  Heads at or past G
    // select nothing.
    SelIn sin;
    if (w < G) select_load(a, row0 + w, lane, sin);   // the histograms are requested before the codes
    uint32_t xr[kGrp][16];
    load_run_group<VEC>(xr, ks, beg, end, tid);
    for (int g = w; g < G; g += 4) {
        if (g != w) select_load(a, row0 + g, lane, sin);
        const ChunkRec r = select_chunk(a, row0 + g, c, lane, sin, s_tr[w]);
        if (lane == 0) {
            s_rec[g][0] = r.off;
            s_rec[g][1] = r.taken;
            s_rec[g][2] = r.ties;
            s_rec[g][3] = r.t;
        }
    }
    __syncthreads();
    uint32_t q[MAXG], nthr[MAXG], nt1[MAXG];
    int off[MAXG], taken[MAXG], mode[MAXG], tie_carry[MAXG];   // mode: 0 no ties, 1 all ties, 2 some ties
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
        const int gg = min(g, G - 1);
        const int* ci = s_rec[gg];
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

// Chunks of whole sub-chunks, at most kMaxChunks per head.  By default about
// topk_wgs workgroups per call: two per CU, so that both scans run in one
// round (their register use allows two workgroups of 256 threads per CU).
int topk_chunk_len(int64_t n, int units) {
    const int64_t per = (int64_t)kSub * kMaxChunks;
    const int64_t min_subs = n > 0 ? (n + per - 1) / per : 1;
    int64_t subs = tuning().topk_subs;
    if (subs <= 0) {
        const int64_t chunks = max((int64_t)1, tuning().topk_wgs / max(units, 1));
        subs = max((int64_t)1, (n + (int64_t)kSub * chunks - 1) / ((int64_t)kSub * chunks));
    }
    return (int)(max(min_subs, subs) * kSub);
}

int topk_hist_row() { return kRow; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    if (a.B <= 0) return hipSuccess;
    if (a.G > 8 || a.chunks > kMaxChunks) return hipErrorInvalidValue;
    if (a.chunks == 0) {
        hipLaunchKernelGGL(k_topk_empty, dim3(a.Hq, a.B), dim3(64), 0, st, a);
        return hipGetLastError();
    }
    if (a.parts > 0) return launch_topk_unit(a, 0, st);
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
    TopkArgs ac = a;
    if (a.q != nullptr) ac.q_sigs = a.q_codes;   // written by the histogram pass
    if (a.G <= 4) {
        if (vec) hipLaunchKernelGGL((k_topk_compact<4, true>), grid, block, 0, st, ac);
        else hipLaunchKernelGGL((k_topk_compact<4, false>), grid, block, 0, st, ac);
    } else {
        if (vec) hipLaunchKernelGGL((k_topk_compact<8, true>), grid, block, 0, st, ac);
        else hipLaunchKernelGGL((k_topk_compact<8, false>), grid, block, 0, st, ac);
    }
    return hipGetLastError();
}

}  // namespace lcda
