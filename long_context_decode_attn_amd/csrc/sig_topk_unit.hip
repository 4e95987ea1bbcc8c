// sig_topk_unit.hip - HashAttention SCORE + TOPK over 32-bit signatures in one
// launch (and, for sparse_decode_step, GATHER-ATT over the selected rows in the
// same launch): the distances are computed once and kept in LDS, and the
// workgroups that share a (batch item, KV head) exchange what they counted.
//
// SCORE(k_i, q) = -popcount(h_i XOR h_q) ("HashAttention: Semantic Sparsity
// for Faster Inference", slide "A 32-bit signature makes scoring cheap",
// Eq. (2)); TOPK keeps the m positions of smallest distance, ties to the lower
// position, united with the first n_sink and last n_recent positions, in
// ascending order (slides "Only selection is approximate; selected KV stay in
// full form" and "Token-level sparsity still needs a careful kernel").
//
// Distances take 33 values, so the top m is fixed by a threshold t and a tie
// quota: every position with d < t is in, and of the positions with d == t the
// lowest `quota` are.
//
// Work unit: one (b, KV head) with its G <= 4 query heads.  Its n positions are
// cut into steps of 4,096, dealt round robin to the unit's Q workgroups (step s
// to workgroup s mod Q, D = 1, 2, 4 or 8 steps each), so that the lowest
// positions - where the tie rule puts the ties it takes, and with them most of
// the selected rows - are spread over all of them.  One workgroup of 16
// wavefronts per (unit, part); the host launches this kernel only when the
// grid fits the device one workgroup per CU.
//   1. Each step's codes are read once (one load instruction of a wavefront
//      covers 1 KB of consecutive codes) and every (position, query head)
//      distance goes into a 33-bin histogram (one LDS copy per lane, so that
//      the 64 increments of one instruction fall into distinct banks; two
//      heads share a copy's word as 16-bit counts) and, as one byte, into the
//      part's LDS distance array, head by head.
//   2. Every workgroup publishes its histograms (cumulative counts, C[d] =
//      positions with distance below d) with device-scope stores and arrives
//      at the unit's counter; the last to arrive releases the others by
//      advancing the unit's epoch word.  One wavefront per query head then
//      finds t and the quota from the summed histograms.
//   3. Each thread owns 4 D consecutive positions of one step and compares
//      their distance bytes, four at a time, with t and t + 1 (byte-parallel
//      subtraction: the bytes are stored as d | 0x80, so the sign bit of byte
//      j of (d | 0x80) - t says whether d_j >= t); dot products with powers of
//      two gather eight sign bits into a byte of the thread's masks.  Per
//      step the workgroup counts the positions below t, the ties and the
//      window positions, and the workgroups exchange these step records the
//      same way; one wavefront per query head (lane = step) turns them into
//      the ties before each step (the ties taken are the lowest ones) and each
//      step's output count and offset.
//   4. Scans of the tie counts and of the selected counts inside each step
//      place every thread's positions; it stores them in order.
// A workgroup that waits too long for its partners (not resident together)
// counts what they publish from the codes itself, so the result never depends
// on co-residency.
// With the rows of the cache (sparse_decode_step) the same workgroups then run
// GATHER-ATT ("HashAttention ...", slide "Only selection is approximate;
// selected KV stay in full form": attention renormalised over the selected
// rows, read straight from the cache by position):
//   5. the part's selected positions of every head also go into an LDS list;
//      16 / G wavefronts per query head walk the head's list, four rows per load
//      instruction (16 lanes per row, 8 values per lane), with an online softmax
//      in base 2, and merge into one partial state (m, l, acc) per head and
//      part;
//   6. the last workgroup of the unit to publish its partial states merges the
//      parts exactly through their maxima (the split identity of the dense path).
// The workspace holds the counters, epochs, histograms and step records; the
// counter words are (tag, arrivals) as for the split pass (see
// arrive_one), so no call needs them cleared, and every call leaves them at
// (tag, 0).

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "sparse.h"
#include "sig_proj.h"

namespace lcda {
namespace {

constexpr int kUT = 1024;                       // threads per workgroup
constexpr int kUW = kUT / 64;                   // wavefronts
constexpr int kStepPos = 4 * kUT;               // positions per step
constexpr int kUBins = 33;
constexpr int kURow = 36;                       // words per published histogram row (34 cumulative counts)
constexpr int kRec = 8;                         // words per step record of a head (7 counts)
constexpr int kMaxSteps = 64;                   // steps per unit (one lane each)
constexpr uint32_t kHi = 0x80808080u;
constexpr uint32_t kPadDist = 0x7Fu;            // distance of a position past the end: never < t, never t

// A step record of one head: its positions below t, its ties (d == t), and
// the sink (ws) and recent (wr) window positions below t and at t.
enum { kBelow = 0, kTies, kWsBelow, kWsTies, kWrBelow, kWrTies, kRecCount };

template <int D>
struct __align__(16) UnitSmem {
    uint32_t dist[4][kUT * D];                  // [head][dword]: the part's distances, a byte d | 0x80 per position
    uint32_t cnt[2 * (kUBins + 1) * 64];        // [head pair][bin][lane]: heads 2p, 2p + 1 in the low and high
                                                // 16 bits; bin 33 takes positions past the end
    uint32_t rec[D][4][kRec];                   // [local step][head] records
    uint32_t s_w[2][kUW];                       // segment scans
    int s_sel[4][2];                            // per head: t, quota
    int s_step[D][4][3];                        // [local step][head]: ties before the step, output offset, count
    int s_total[4];
    uint32_t s_code[4];
    int s_flag;
};

__device__ __forceinline__ uint32_t scan_incl(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return x;
}

__device__ __forceinline__ uint32_t lane_val(uint32_t x, int l) {   // l uniform
    return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}

__device__ __forceinline__ uint32_t wave_total(uint32_t x) { return lane_val(scan_incl(x), 63); }

// Exclusive prefixes of x0 and x1 over the threads of the calling thread's
// segment: the run of whole wavefronts from wavefront seg0 to the next
// segment's first.  Ends with a barrier after its last LDS read.
__device__ __forceinline__ void seg_scan2(uint32_t x0, uint32_t x1, int seg0, uint32_t (*s_w)[kUW], uint32_t& e0,
                                          uint32_t& e1) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t i0 = scan_incl(x0), i1 = scan_incl(x1);
    if (lane == 63) {
        s_w[0][w] = i0;
        s_w[1][w] = i1;
    }
    __syncthreads();
    uint32_t b0 = 0, b1 = 0;
#pragma unroll
    for (int k = 0; k < kUW; ++k) {
        const bool in = k >= seg0 && k < w;
        b0 += in ? s_w[0][k] : 0u;
        b1 += in ? s_w[1][k] : 0u;
    }
    __syncthreads();
    e0 = b0 + i0 - x0;
    e1 = b1 + i1 - x1;
}

// Dword dw of a head's distance array (local positions 4 dw .. 4 dw + 3; local
// step dw / 1024): thread T of the compaction owns dwords D T .. D T + D - 1.
// With D = 8 (two 16-byte chunks per thread) the chunks of a thread are
// swapped for odd T / 8, so that 16 neighbouring threads' reads of one chunk
// each fall into distinct banks.
template <int D>
__device__ __forceinline__ int dist_slot(int dw) {
    if (D != 8) return dw;
    const int c = dw >> 2, t = c >> 1;
    return (((t << 1) | ((c & 1) ^ ((t >> 3) & 1))) << 2) | (dw & 3);
}

// Bits 0 .. 31 below c (c clamped to 0 .. 32).
__device__ __forceinline__ uint32_t low_bits(int64_t c) {
    return c <= 0 ? 0u : (c >= 32 ? 0xFFFFFFFFu : ((1u << (int)c) - 1u));
}

// Bits 8 k .. 8 k + 7 = flags of positions 8 k .. 8 k + 7 for two dwords of
// distance bytes (each byte d | 0x80), 4 k and 4 k + 1 of the thread: bit 7 of
// byte e of ~(A - T) is set iff d_e < t.  Two dot products with weights
// 1, 2, 4, 8 and 16, 32, 64, 128 gather the eight sign bits as 128 x byte.
__device__ __forceinline__ uint32_t below8(uint32_t A0, uint32_t A1, uint32_t T, bool two) {
    uint32_t r = __builtin_amdgcn_udot4(~(A0 - T) & kHi, 0x08040201u, 0u, false);
    if (two) r = __builtin_amdgcn_udot4(~(A1 - T) & kHi, 0x80402010u, r, false);
    return r;   // 128 x the 8 flags
}

// Global step of local step ls of workgroup `part` (of Q).
__device__ __forceinline__ int global_step(int ls, int Q, int part) { return ls * Q + part; }

// The window positions are [0, s_end) and [r_beg, n): every one of them is
// selected, for every head, and they take the first s_end and the last
// n - r_beg entries of each index list.  The unit's workgroups share them out
// in contiguous runs [w0, w1) of the window sequence (k -> k below s_end, else
// r_beg + k - s_end).
struct Windows {
    int s_end, r_beg, n;
    int w0, w1;   // this workgroup's run
    __device__ __forceinline__ int count() const { return s_end + (n - r_beg); }
    __device__ __forceinline__ int pos(int k) const { return k < s_end ? k : r_beg + (k - s_end); }
    // Window positions of global step gs: the sink portion (a prefix of the
    // step) and the recent portion (a suffix).
    __device__ __forceinline__ int sink_in(int gs) const {
        const int sb = gs * kStepPos, se = min(n, sb + kStepPos);
        return max(0, min(se, s_end) - sb);
    }
    __device__ __forceinline__ int recent_in(int gs) const {
        const int sb = gs * kStepPos, se = min(n, sb + kStepPos);
        return max(0, se - max(sb, r_beg));
    }
};

// Thread 0 of one of the unit's Q workgroups, once the workgroup's published
// stores are acknowledged: arrival at counter c and, but for the last to
// arrive, a wait of at most spin_max polls for the epoch word ep to move on
// from e, the value it held before any of them arrived (the last arrival
// advances it).  Returns whether the workgroup was released.
__device__ __forceinline__ int arrive_wait(unsigned long long* c, uint32_t* ep, uint32_t e, uint32_t Q, int spin_max) {
    if (arrive_one(c, Q) == Q) {
        __hip_atomic_store(ep, e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return 1;
    }
    for (int it = 0; it < spin_max; ++it) {
        if (__hip_atomic_load(ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != e) return 1;
        __builtin_amdgcn_s_sleep(1);
    }
    return 0;
}

template <int D>
__device__ __forceinline__ void zero_counts(UnitSmem<D>& sm) {
    for (int k = threadIdx.x; k < 2 * (kUBins + 1) * 64; k += kUT) sm.cnt[k] = 0u;
}

// Histograms of part p's steps for heads g < G, counted from the codes into the
// LDS copies (zeroed by the caller): the fallback of a workgroup whose
// partners did not arrive in time.
template <int D>
__device__ void count_part(const TopkArgs& a, UnitSmem<D>& sm, const uint32_t* ks, const uint32_t (&q)[4], int p) {
    const int lane = threadIdx.x & 63;
    const int n = (int)a.n;
    for (int ls = 0; ls < D; ++ls) {
        const int beg = global_step(ls, a.parts, p) * kStepPos;
        for (int i = beg + (int)threadIdx.x; i < min(n, beg + kStepPos); i += kUT) {
            const uint32_t x = ks[i];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g < a.G) {
                    const uint32_t d = (uint32_t)__builtin_popcount(x ^ q[g]);
                    __hip_atomic_fetch_add(&sm.cnt[(((g >> 1) * (kUBins + 1) + d) << 6) + lane], 1u << (16 * (g & 1)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        }
    }
}

// Publish the histograms in the LDS copies as cumulative counts: row g of prow
// ([head][kURow]) gets C[d], d = 0 .. 33.  Wavefront g (lane = bin) sums the
// bin over the lane copies and scans over the bins.
template <int D>
__device__ __forceinline__ void publish_hist(const TopkArgs& a, const UnitSmem<D>& sm, uint32_t* prow) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (w >= 4) return;
    uint32_t v = 0;
    if (w < a.G && lane < kUBins) {
        const uint32_t* r = sm.cnt + (((w >> 1) * (kUBins + 1) + lane) << 6);
        const int sh = 16 * (w & 1);
#pragma unroll 8
        for (int c = 0; c < 64; ++c) v += (r[(c + lane) & 63] >> sh) & 0xFFFFu;   // lane-rotated: distinct banks
    }
    const uint32_t incl = scan_incl(v);
    uint32_t* row = prow + w * kURow;
    if (lane < kUBins) store_dev(row + lane + 1, incl);
    if (lane == 0) store_dev(row, 0u);
}

// Adds the calling wavefront's share of a step record (per head g < G: bit
// masks of positions below t and at t, and the window masks) to rec[g], with
// one LDS atomic per count.  Every lane of the wavefront takes part; its
// positions lie in one step.  The window counts are only summed in the
// wavefronts that hold window positions.
__device__ __forceinline__ void add_records(uint32_t (*rec)[kRec], int G, const uint32_t* lt4, const uint32_t* eq4,
                                            uint32_t ws, uint32_t wr) {
    const bool anyw = __builtin_amdgcn_ballot_w64((ws | wr) != 0u) != 0;   // uniform
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (g < G) {
            const uint32_t l = lt4[g], e = eq4[g];
            const uint32_t s0 = wave_total((uint32_t)__builtin_popcount(l) | ((uint32_t)__builtin_popcount(e) << 16));
            uint32_t s1 = 0, s2 = 0;
            if (anyw) {
                s1 = wave_total((uint32_t)__builtin_popcount(l & ws) | ((uint32_t)__builtin_popcount(e & ws) << 16));
                s2 = wave_total((uint32_t)__builtin_popcount(l & wr) | ((uint32_t)__builtin_popcount(e & wr) << 16));
            }
            if ((threadIdx.x & 63) == 0) {
                uint32_t* r = rec[g];
                __hip_atomic_fetch_add(r + kBelow, s0 & 0xFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(r + kTies, s0 >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (anyw) {
                    __hip_atomic_fetch_add(r + kWsBelow, s1 & 0xFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_fetch_add(r + kWsTies, s1 >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_fetch_add(r + kWrBelow, s2 & 0xFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_fetch_add(r + kWrTies, s2 >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        }
    }
}

// Rows of 128 values as 8 floats per lane (16 lanes per row).
template <typename T>
struct GRow;
template <>
struct GRow<float> {
    u32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = ld16_nt(p);
        b = ld16_nt(p + 4);
    }
    __device__ __forceinline__ void to_float(float (&x)[8]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = __uint_as_float(a[e]);
            x[4 + e] = __uint_as_float(b[e]);
        }
    }
};
template <>
struct GRow<uint16_t> {
    u32x4 a;
    __device__ __forceinline__ void load(const uint16_t* p) { a = ld16_nt(p); }
    __device__ __forceinline__ void to_float(float (&x)[8]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(a[e]);
            x[2 * e + 1] = bf16_hi(a[e]);
        }
    }
};

// The arguments combine_row reads: the parts' partial states of a query row.
struct PartMerge {
    int splits;
    const float2* ml;
    const float* acc;
    const float* alpha_in;
    const float* a_in;
    float* out;
    float* alpha;
};

// GATHER-ATT over this part's share of the selected positions of each query
// head, then the merge of the parts (see the file comment, steps 5 and 6).
// Head g's share: the part's cntg[g] selected positions outside the windows,
// local step by local step - in LDS from lbase[g] (local position numbers
// 4096 ls + offset in the step) when in_lds, else in the index list at each
// local step's output offset past its sink portion - then the part's run of
// window positions.
template <typename T, int D>
__device__ void gather_part(const TopkArgs& a, UnitSmem<D>& sm, const uint16_t* lst, bool in_lds, const int (&cntg)[4],
                            const int (&lbase)[4], const Windows& win, int unit, int part, int64_t row0, int b, int h) {
    constexpr int U = sizeof(T) == 2 ? 4 : 2;   // rows per lane group and step (fewer for fp32 rows)
    constexpr int kStep = 4 * U;                 // rows per wavefront and step
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront-uniform values in scalar registers
    const int j = lane >> 4, c16 = lane & 15;
    const int G = a.G, Q = a.parts;
    const int Wh = kUW / G;              // wavefronts per head (G <= 4)
    const int gw = w / Wh, wi = w % Wh;  // this wavefront's head (gw >= G: idle) and its rank
    float m = kNoMax, l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (gw < G) {
        const int64_t row = row0 + gw;
        const int own = __builtin_amdgcn_readfirstlane(gw == 0 ? cntg[0] : gw == 1 ? cntg[1] : gw == 2 ? cntg[2] : cntg[3]);
        const int wbeg = __builtin_amdgcn_readfirstlane(win.w0 - own);   // entry t >= own: window entry wbeg + t
        const int cnt = own + (win.w1 - win.w0);
        const int lb = __builtin_amdgcn_readfirstlane(gw == 0 ? lbase[0] : gw == 1 ? lbase[1] : gw == 2 ? lbase[2] : lbase[3]);
        const int64_t head = (a.kv_batch_stride == 0 ? 0 : (int64_t)b * a.kv_batch_stride) + (int64_t)h * a.n * kD;
        const T* kh = static_cast<const T*>(a.gk) + head + 8 * c16;
        const T* vh = static_cast<const T*>(a.gv) + head + 8 * c16;
        const uint32_t* ilist = reinterpret_cast<const uint32_t*>(a.idx + row * a.cap);
        float qv[8];
        {
            GRow<T> x;
            x.load(static_cast<const T*>(a.gq) + row * kD + 8 * c16);
            x.to_float(qv);
        }
        struct Step {
            GRow<T> k[U], v[U];
        };
        // Own entry t of the head's list -> its position, from the index list
        // the workgroup has written (a list too long for LDS).
        auto from_idx = [&](int t) -> int {
            int ls = 0, base = 0;
#pragma unroll
            for (int k = 0; k < D - 1; ++k) {
                const int gs = global_step(k, Q, part);
                const int c = sm.s_step[k][gw][2] - win.sink_in(gs) - win.recent_in(gs);   // 0 past the end
                if (ls == k && t >= base + c) {
                    ls = k + 1;
                    base += c;
                }
            }
            const int gs = global_step(ls, Q, part);
            return (int)load_dev_u32(ilist + sm.s_step[ls][gw][1] + win.sink_in(gs) + (t - base));
        };
        // The rows of entries t0 + 4 u + j of the list (clamped to the last
        // entry; rows past cnt are masked in compute).
        auto fetch = [&](Step& st, int t0, auto listed) {
            int pos[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = min(t0 + 4 * u + j, cnt - 1);
                if (t >= own) {
                    pos[u] = win.pos(wbeg + t);
                } else if constexpr (decltype(listed)::value) {
                    const int loc = (int)lst[lb + t];
                    pos[u] = global_step(loc >> 12, Q, part) * kStepPos + (loc & (kStepPos - 1));
                } else {
                    pos[u] = from_idx(t);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                st.k[u].load(kh + (int64_t)pos[u] * kD);
                st.v[u].load(vh + (int64_t)pos[u] * kD);
            }
        };
        auto compute = [&](const Step& st, int t0) {
            float s[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[8];
                st.k[u].to_float(kf);
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qv[e], kf[e], d);
                d = sum16(d) * a.scale_log2;
                s[u] = t0 + 4 * u + j < cnt ? d : -INFINITY;
            }
            float bm = s[0];
#pragma unroll
            for (int u = 1; u < U; ++u) bm = fmaxf(bm, s[u]);
            const float mn = fmaxf(m, bm);
            const float sc = fast_exp2(m - mn);
            m = mn;
            l *= sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[8];
                st.v[u].to_float(vf);
                const float p = fast_exp2(s[u] - m);
                l += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
            }
        };
        // Software pipeline: the rows of the next step are requested before the
        // current step is computed, unconditionally (entries past the list are
        // clamped to its last one), so that waiting for the current step's rows
        // never waits for the next step's.
        auto walk = [&](auto listed) {
            int t0 = wi * kStep;
            const int stride = Wh * kStep;
            if (t0 >= cnt) return;
            Step s0, s1;
            fetch(s0, t0, listed);
            while (true) {
                fetch(s1, t0 + stride, listed);
                compute(s0, t0);
                t0 += stride;
                if (t0 >= cnt) break;
                fetch(s0, t0 + stride, listed);
                compute(s1, t0);
                t0 += stride;
                if (t0 >= cnt) break;
            }
        };
        if (in_lds) walk(std::true_type{});
        else walk(std::false_type{});
    }
    // Merge the 4 lane groups of the wavefront, then the head's wavefronts
    // through LDS (the counters' space is free now).
    {
        const float M = max_xor32(max_xor16(m));
        const float wt = fast_exp2(m - M);
        const float L = sum_xor32(sum_xor16(l * wt));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = sum_xor32(sum_xor16(acc[e] * wt));
        float* so = reinterpret_cast<float*>(sm.cnt);          // [kUW][kD] sums
        float2* sml = reinterpret_cast<float2*>(so + kUW * kD); // [kUW] (m, l)
        if (j == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) so[w * kD + 8 * c16 + e] = acc[e];
            if (c16 == 0) sml[w] = make_float2(M, L);
        }
        __syncthreads();
        // Wavefront wi == 0 of head gw: the part's state of the head (lane:
        // columns 2 lane, 2 lane + 1), published for the merge of the parts.
        if (gw < G && wi == 0) {
            float Mx = kNoMax;
            for (int k = 0; k < Wh; ++k) Mx = fmaxf(Mx, sml[w + k].x);
            float Lx = 0.f, x0 = 0.f, x1 = 0.f;
            for (int k = 0; k < Wh; ++k) {
                const float2 ml = sml[w + k];
                const float f = ml.y > 0.f ? fast_exp2(ml.x - Mx) : 0.f;
                Lx += f * ml.y;
                x0 += f * so[(w + k) * kD + 2 * lane];
                x1 += f * so[(w + k) * kD + 2 * lane + 1];
            }
            const int64_t slot = (row0 + gw) * Q + part;
            if (Q == 1) {   // one part: the row is finished here
                const bool has = Lx > 0.f;
                const float r = has ? 1.f / Lx : 0.f;
                a.out[(row0 + gw) * kD + 2 * lane] = x0 * r;
                a.out[(row0 + gw) * kD + 2 * lane + 1] = x1 * r;
                if (a.alpha && lane == 0) a.alpha[row0 + gw] = has ? (Mx + log2f(Lx)) * kLn2 : -INFINITY;
            } else {
                store_dev(a.pacc + slot * kD + 2 * lane, x0);
                store_dev(a.pacc + slot * kD + 2 * lane + 1, x1);
                if (lane == 0) store_dev(a.pml + slot, make_float2(Mx, Lx));
            }
        }
    }
    if (Q == 1) return;
    // ---- 6. the last workgroup of the unit merges the parts ----------------------------------
    if (!arrive_count(a.bar2 + unit, (uint32_t)Q, &sm.s_flag)) return;
    const int wv = tid >> 6;
    if (wv < G) {
        PartMerge pm{Q, a.pml, a.pacc, nullptr, nullptr, a.out, a.alpha};
        combine_row(pm, row0 + wv, lane);
    }
}

// D: steps of 4,096 positions per workgroup (1024 D dwords of distances per
// head).  T: the rows' type for the fused GATHER-ATT (float or uint16_t for
// bf16), void for TOPK alone.
template <int D, bool SCORES, typename T>
__global__ __launch_bounds__(kUT) void k_topk_unit(TopkArgs a) {
    constexpr bool kGather = !std::is_void<T>::value;
    __shared__ UnitSmem<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int Q = a.parts;
    // Workgroup -> (unit, part): part-major, so that with a multiple of 8 units
    // the parts of a unit run on one XCD (workgroups go round the 8 XCDs in
    // turn).
    const int units = a.B * a.Hkv;
    const int unit = blockIdx.x % units, part = blockIdx.x / units;
    const int b = unit / a.Hkv, h = unit % a.Hkv;
    const int G = a.G;
    const int n = (int)a.n;
    const int NS = (n + kStepPos - 1) / kStepPos;   // the unit's steps (<= kMaxSteps)
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int64_t row0 = (int64_t)b * a.Hq + (int64_t)h * G;
    const int s_end = (int)min(a.n_sink, a.n);
    const int r_beg = (int)max((int64_t)s_end, a.n - a.n_recent);
    const bool vec = (n & 3) == 0;   // uniform
    // Thread 0: the exchanges' epochs as they stand before this call's arrivals.
    uint32_t e_hist = 0, e_rec = 0;
    if (tid == 0 && Q > 1) {
        e_hist = __hip_atomic_load(a.epoch + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        e_rec = __hip_atomic_load(a.repoch + unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- 1. distances ------------------------------------------------------------------
    // The query codes first (so that waiting for them is not waiting for all the
    // codes), then local step ls: positions 4096 global_step(ls) + 4 tid + e,
    // e < 4; every step's codes are requested at once.
    uint32_t q[4];
    if (a.q == nullptr) {
#pragma unroll
        for (int g = 0; g < 4; ++g) q[g] = a.q_sigs[row0 + min(g, G - 1)];
    }
    u32x4 xc[D];
#pragma unroll
    for (int ls = 0; ls < D; ++ls) {
        const int i = global_step(ls, Q, part) * kStepPos + 4 * tid;
        if (vec) {
            xc[ls] = ld16(ks + min(i, n - 4));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) xc[ls][e] = ks[min(i + e, n - 1)];
        }
    }
    if (a.q != nullptr) {   // uniform: the query codes are encoded here (T_map), while the codes load
        static_assert(sizeof(sm.dist) + sizeof(sm.cnt) >= (kD * 32 + 4 * kD) * 4,
                      "R and the query rows fit the distances' and counters' LDS");
        float* sR = reinterpret_cast<float*>(&sm.dist[0][0]);
        float* sQ = sR + kD * 32;
        for (int k = tid; k < kD * 32; k += kUT) {
            const int e = k >> 5, bit = k & 31;
            sR[k] = bit < a.bits ? a.R[e * a.bits + bit] : 0.f;
        }
        for (int k = tid; k < G * kD; k += kUT) {
            const int64_t i = row0 * kD + k;
            sQ[k] = a.q_bf16 ? bf16_lo(static_cast<const uint16_t*>(a.q)[i]) : static_cast<const float*>(a.q)[i];
        }
        __syncthreads();
        if (tid < 32 * G) {
            const int g = tid >> 5, bit = tid & 31;
            const double z = proj_chain([&](int e) { return sQ[g * kD + e]; }, sR + bit, 32);
            const uint64_t bits = __ballot(z > 0.0);
            if ((tid & 31) == 0) sm.s_code[g] = (uint32_t)(bits >> (tid & 32));
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < 4; ++g) q[g] = sm.s_code[min(g, G - 1)];
        if (part == 0 && tid < G) a.q_codes[row0 + tid] = sm.s_code[tid];
        __syncthreads();   // the staging area is about to hold distances
    }
    zero_counts(sm);
    for (int k = tid; k < D * 4 * kRec; k += kUT) (&sm.rec[0][0][0])[k] = 0u;
    __syncthreads();

    uint32_t* mycnt = sm.cnt + lane;
#pragma unroll
    for (int ls = 0; ls < D; ++ls) {
        const int gs = global_step(ls, Q, part);
        const int i = gs * kStepPos + 4 * tid;
        const int dw = dist_slot<D>(kUT * ls + tid);
        if ((gs + 1) * kStepPos <= n) {   // uniform: every position of the step is below n
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g < G) {   // uniform
                    uint32_t pk = kHi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t d = (uint32_t)__builtin_popcount(xc[ls][e] ^ q[g]);
                        __hip_atomic_fetch_add(mycnt + (((g >> 1) * (kUBins + 1) + d) << 6), 1u << (16 * (g & 1)),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        pk |= d << (8 * e);
                        if (SCORES) a.scores[(row0 + g) * a.n + i + e] = (int8_t)(-(int)d);
                    }
                    sm.dist[g][dw] = pk;
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g < G) {
                    uint32_t pk = kHi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = i + e < n;
                        const uint32_t d = ok ? (uint32_t)__builtin_popcount(xc[ls][e] ^ q[g]) : (uint32_t)kUBins;
                        __hip_atomic_fetch_add(mycnt + (((g >> 1) * (kUBins + 1) + d) << 6), 1u << (16 * (g & 1)),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        pk |= (ok ? d : kPadDist) << (8 * e);
                        if (SCORES && ok) a.scores[(row0 + g) * a.n + i + e] = (int8_t)(-(int)d);
                    }
                    sm.dist[g][dw] = pk;
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. histogram exchange, threshold and quota ---------------------------------------
    uint32_t* phist = a.phist + (int64_t)unit * Q * 4 * kURow;
    publish_hist(a, sm, phist + (int64_t)part * 4 * kURow);
    if (Q > 1) {
        wait_vm_all();      // this thread's histogram stores are acknowledged
        __syncthreads();    // ... in every thread
        if (tid == 0) sm.s_flag = arrive_wait(a.bar + unit, a.epoch + unit, e_hist, (uint32_t)Q, a.spin_max);
        __syncthreads();
        if (!sm.s_flag) {   // uniform: the partners did not arrive in time; count their parts here
            for (int p = 0; p < Q; ++p) {
                if (p == part) continue;
                zero_counts(sm);
                __syncthreads();
                count_part(a, sm, ks, q, p);
                __syncthreads();
                publish_hist(a, sm, phist + (int64_t)p * 4 * kURow);
                __syncthreads();
            }
        }
    }
    wait_vm_all();
    __syncthreads();
    if (w < G) {   // one wavefront per query head
        const int g = w;
        // Lane d: S[d] = the unit's positions with distance <= d; the requests
        // of up to 8 parts are issued together.
        uint32_t S = 0;
        if (lane < kUBins) {
            for (int p0 = 0; p0 < Q; p0 += 8) {
                uint32_t v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    v[k] = p0 + k < Q ? load_dev_u32(phist + ((int64_t)(p0 + k) * 4 + g) * kURow + lane + 1) : 0u;
#pragma unroll
                for (int k = 0; k < 8; ++k) S += v[k];
            }
        }
        const uint32_t meff = (uint32_t)min(a.m, a.n);
        const uint64_t reach = __ballot(lane < kUBins && meff > 0 && S >= meff);
        const int t = reach ? (int)__builtin_ctzll(reach) : -1;
        const uint32_t below_all = t > 0 ? lane_val(S, t - 1) : 0u;
        if (lane == 0) {
            sm.s_sel[g][0] = t;
            sm.s_sel[g][1] = t >= 0 ? (int)(meff - below_all) : 0;
        }
    }
    __syncthreads();

    // ---- 3. masks, step records and their exchange ------------------------------------------
    // Thread tid: local dwords D tid .. D tid + D - 1, all in local step ls_me;
    // bit j of its masks is position P0 + j.
    const int ls_me = (D * tid) >> 10;
    const int P0 = global_step(ls_me, Q, part) * kStepPos + 4 * ((D * tid) & 1023);
    int tg[4];
    uint32_t lt[4], eq[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        lt[g] = eq[g] = 0u;
        tg[g] = -1;
        if (g < G) {
            const int t = sm.s_sel[g][0];
            tg[g] = t;
            const uint32_t T0 = t >= 0 ? (uint32_t)t * 0x01010101u : 0u;   // t = -1 (m = 0): nothing below
            const uint32_t T1 = t >= 0 ? (uint32_t)(t + 1) * 0x01010101u : 0u;
            uint32_t l = 0, le = 0;
#pragma unroll
            for (int j = 0; j < D; j += 2) {
                const uint32_t A0 = sm.dist[g][dist_slot<D>(D * tid + j)];
                const uint32_t A1 = j + 1 < D ? sm.dist[g][dist_slot<D>(D * tid + j + 1)] : 0u;
                const uint32_t r0 = below8(A0, A1, T0, j + 1 < D), r1 = below8(A0, A1, T1, j + 1 < D);
                l |= j == 0 ? r0 >> 7 : r0 << (4 * j - 7);
                le |= j == 0 ? r1 >> 7 : r1 << (4 * j - 7);
            }
            lt[g] = l;
            eq[g] = le & ~l;
        }
    }
    const uint32_t vmask = low_bits(n - P0) & low_bits(4 * D);
    const uint32_t wsm = low_bits(s_end - P0) & vmask;
    const uint32_t wrm = ~low_bits(r_beg - P0) & vmask;
    add_records(sm.rec[ls_me], G, lt, eq, wsm, wrm);
    __syncthreads();
    uint32_t* grec = a.srec + (int64_t)unit * kMaxSteps * 4 * kRec;   // [global step][head][kRec]
    for (int k = tid; k < D * 4 * kRec; k += kUT) {
        const int ls = k / (4 * kRec), rest = k % (4 * kRec);
        const int gs = global_step(ls, Q, part);
        if (gs < NS) store_dev(grec + (int64_t)gs * 4 * kRec + rest, (&sm.rec[ls][0][0])[rest]);
    }
    if (Q > 1) {
        wait_vm_all();
        __syncthreads();
        if (tid == 0) sm.s_flag = arrive_wait(a.rbar + unit, a.repoch + unit, e_rec, (uint32_t)Q, a.spin_max);
        __syncthreads();
        if (!sm.s_flag) {   // uniform: count the other workgroups' steps here, four positions per thread
            for (int gs = 0; gs < NS; ++gs) {
                if (gs % Q == part) continue;
                for (int k = tid; k < 4 * kRec; k += kUT) (&sm.rec[0][0][0])[k] = 0u;
                __syncthreads();
                const int p0 = gs * kStepPos + 4 * tid;
                uint32_t l4[4], e4[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    l4[g] = e4[g] = 0u;
                    if (g < G && tg[g] >= 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (p0 + e < n) {
                                const int d = __builtin_popcount(ks[p0 + e] ^ q[g]);
                                l4[g] |= (d < tg[g] ? 1u : 0u) << e;
                                e4[g] |= (d == tg[g] ? 1u : 0u) << e;
                            }
                        }
                    }
                }
                const uint32_t vm = low_bits(n - p0) & 0xFu;
                add_records(sm.rec[0], G, l4, e4, low_bits(s_end - p0) & vm, ~low_bits(r_beg - p0) & vm);
                __syncthreads();
                for (int k = tid; k < 4 * kRec; k += kUT)
                    store_dev(grec + (int64_t)gs * 4 * kRec + k, (&sm.rec[0][0][0])[k]);
                __syncthreads();
            }
        }
    }
    wait_vm_all();
    __syncthreads();
    // One wavefront per query head, lane = global step: the ties before each
    // step, the ties it takes, its output count and offset.
    if (w < G) {
        const int g = w;
        const uint32_t quota = (uint32_t)sm.s_sel[g][1];
        uint32_t r[kRecCount];
#pragma unroll
        for (int k = 0; k < kRecCount; ++k)
            r[k] = lane < NS ? load_dev_u32(grec + ((int64_t)lane * 4 + g) * kRec + k) : 0u;
        const uint32_t ties = r[kTies];
        const uint32_t ties_before = scan_incl(ties) - ties;
        const uint32_t taken = quota > ties_before ? min(quota - ties_before, ties) : 0u;
        // The ties a step takes are its lowest ones: its sink window portion (a
        // prefix of the step) holds the first of them, its recent portion (a
        // suffix) what is left after the ties before that portion.
        const uint32_t tk_s = min(r[kWsTies], taken);
        const uint32_t tk_r = taken > ties - r[kWrTies] ? min(taken - (ties - r[kWrTies]), r[kWrTies]) : 0u;
        // The step's window positions: its sink and recent portions.
        const int sb = lane * kStepPos, se = min(n, sb + kStepPos);
        const uint32_t win_n = lane < NS ? (uint32_t)(max(0, min(se, s_end) - sb) + max(0, se - max(sb, r_beg))) : 0u;
        const uint32_t cnt = r[kBelow] + taken + win_n - (r[kWsBelow] + tk_s + r[kWrBelow] + tk_r);
        const uint32_t cincl = scan_incl(cnt);
        const uint32_t total = lane_val(cincl, 63);
#pragma unroll
        for (int ls = 0; ls < D; ++ls) {   // every lane takes part in the reads (readlane outside divergent code)
            const int gs = global_step(ls, Q, part);
            const int gl = min(gs, kMaxSteps - 1);
            const uint32_t tb = lane_val(ties_before, gl), off = lane_val(cincl - cnt, gl), c = lane_val(cnt, gl);
            if (lane == 0) {
                sm.s_step[ls][g][0] = (int)tb;
                sm.s_step[ls][g][1] = (int)off;
                sm.s_step[ls][g][2] = gs < NS ? (int)c : 0;
            }
        }
        if (lane == 0) sm.s_total[g] = (int)total;
    }
    __syncthreads();

    // ---- 4. ordered compaction --------------------------------------------------------------
    const int seg0 = (ls_me * (kUT / D)) >> 6;   // first wavefront of this thread's step
    uint32_t te01, te23;
    {
        uint32_t tv[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) tv[g] = (uint32_t)__builtin_popcount(eq[g]);
        seg_scan2(tv[0] | (tv[1] << 16), tv[2] | (tv[3] << 16), seg0, sm.s_w, te01, te23);
    }
    const uint32_t winm = wsm | wrm;
    uint32_t sel[4], nsel[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        sel[g] = nsel[g] = 0u;
        if (g < G) {
            const uint32_t ties = (uint32_t)__builtin_popcount(eq[g]);
            const uint32_t local = ((g < 2 ? te01 : te23) >> (16 * (g & 1))) & 0xFFFFu;
            const uint32_t before = (uint32_t)sm.s_step[ls_me][g][0] + local;
            const uint32_t quota = (uint32_t)sm.s_sel[g][1];
            const uint32_t take = quota > before ? min(quota - before, ties) : 0u;
            uint32_t tk = 0;
            if (take == ties) {
                tk = eq[g];
            } else {   // the one thread where the quota ends: its lowest `take` ties
                uint32_t e = eq[g];
                for (uint32_t k = 0; k < take; ++k) {
                    const uint32_t low = e & (0u - e);
                    tk |= low;
                    e ^= low;
                }
            }
            sel[g] = lt[g] | tk | winm;
            nsel[g] = __builtin_popcount(sel[g]);
        }
    }
    uint32_t oe01, oe23;
    seg_scan2(nsel[0] | (nsel[1] << 16), nsel[2] | (nsel[3] << 16), seg0, sm.s_w, oe01, oe23);
    // The window positions' entries are stored by all the unit's workgroups,
    // each its run of them; a thread stores its other selected positions.  The
    // part's selected positions of head g outside the windows, cntg[g] of them,
    // are also listed in LDS (local position numbers, after the lists of the
    // heads before) when they fit.  The distance array is no longer read.
    Windows win;
    win.s_end = s_end;
    win.r_beg = r_beg;
    win.n = n;
    win.w0 = (int)((int64_t)win.count() * part / Q);
    win.w1 = (int)((int64_t)win.count() * (part + 1) / Q);
    int cntg[4], lbase[4];
    int lsum = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        int c = 0;
#pragma unroll
        for (int ls = 0; ls < D; ++ls) {
            const int gs = global_step(ls, Q, part);
            c += g < G && gs < NS ? sm.s_step[ls][g][2] - win.sink_in(gs) - win.recent_in(gs) : 0;
        }
        cntg[g] = c;
        lbase[g] = lsum;
        lsum += c;
    }
    uint16_t* lst = reinterpret_cast<uint16_t*>(&sm.dist[0][0]);
    const bool in_lds = kGather && lsum <= (int)(sizeof(sm.dist) / 2);   // uniform
    const int loc0 = 4 * D * tid;   // local position number of bit 0 (local step ls_me = loc0 >> 12)
    // Window positions of this thread's step before P0.
    const int sb_me = global_step(ls_me, Q, part) * kStepPos;
    const int wpre = max(0, min(P0, s_end) - sb_me) + max(0, P0 - max(sb_me, r_beg));
    const uint32_t other = ~winm;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (g < G) {
            int32_t* out = a.idx + (row0 + g) * a.cap;
            const int total = sm.s_total[g];
            const uint32_t local = ((g < 2 ? oe01 : oe23) >> (16 * (g & 1))) & 0xFFFFu;
            // Stores through a buffer resource bounded to the row's first
            // min(cap, n) entries (the count is at most both).
            const __amdgpu_buffer_rsrc_t ro =
                __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)(min(a.cap, a.n) * 4), kRsrcWord3);
            const uint32_t base4 = 4u * ((uint32_t)sm.s_step[ls_me][g][1] + local);
            int li = lbase[g] + (int)local - wpre;   // after this head's entries of the local steps before
#pragma unroll
            for (int ls = 0; ls < D; ++ls) {
                const int gs = global_step(ls, Q, part);
                li += ls < ls_me ? sm.s_step[ls][g][2] - win.sink_in(gs) - win.recent_in(gs) : 0;
            }
            const uint32_t sg = sel[g];
            uint32_t s = sg & other;
            while (s) {
                const int bit = __builtin_ctz(s);
                const uint32_t below = (uint32_t)__builtin_popcount(sg & ((1u << bit) - 1u));
                __builtin_amdgcn_raw_buffer_store_b32(P0 + bit, ro, base4 + 4u * below, 0, 0);
                if (in_lds) lst[li++] = (uint16_t)(loc0 + bit);
                s &= s - 1u;
            }
            // This workgroup's run of window entries: the sink portion at the
            // head of the list, the recent portion at its end.
            for (int k = win.w0 + tid; k < win.w1; k += kUT) {
                const int o = k < s_end ? k : total - (n - r_beg) + (k - s_end);
                __builtin_amdgcn_raw_buffer_store_b32(win.pos(k), ro, 4u * (uint32_t)o, 0, 0);
            }
            if (part == 0) {
                if (tid == 0) a.count[row0 + g] = total;
                for (int64_t i = (int64_t)total + tid; i < a.cap; i += kUT) out[i] = -1;
            }
        }
    }
    if constexpr (kGather) {
        if (!in_lds) wait_vm_all();   // the index stores are acknowledged: the list is read back from them
        __syncthreads();
        gather_part<T>(a, sm, lst, in_lds, cntg, lbase, win, unit, part, row0, b, h);
    }
}

}  // namespace

// Positions per part for a unit of n positions when `units` units share the
// device's `cus` compute units: D steps of 4,096 positions (D = 1, 2, 4, 8),
// the smallest D with units * ceil(steps / D) <= cus; 0 when none fits, G > 4,
// or the unit has more than kMaxSteps steps.
int topk_unit_part(int64_t n, int units, int G, int cus) {
    if (n <= 0 || G > 4 || units <= 0) return 0;
    const int64_t steps = (n + kStepPos - 1) / kStepPos;
    if (steps > kMaxSteps) return 0;
    for (int D = 1; D <= 8; D *= 2) {
        const int64_t parts = (steps + D - 1) / D;
        if ((int64_t)units * parts <= cus) return kStepPos * D;
    }
    return 0;
}

int topk_unit_row_words() { return kURow; }
int topk_unit_rec_words() { return kMaxSteps * 4 * kRec; }

hipError_t launch_topk_unit(const TopkArgs& a, int dtype, hipStream_t st) {
    const int D = a.part_len / kStepPos;
    if (a.B <= 0 || a.G > 4 || a.parts <= 0 || a.part_len != kStepPos * D || (D != 1 && D != 2 && D != 4 && D != 8) ||
        a.n <= 0 || (a.n + kStepPos - 1) / kStepPos > kMaxSteps || a.parts != (int)((a.n + a.part_len - 1) / a.part_len))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.B * a.Hkv * a.parts)), block(kUT);
    const bool sc = a.scores != nullptr;
    const int kind = a.gk == nullptr ? 0 : (dtype == 0 ? 1 : 2);
#define LCDA_UNIT3(DD, SC, TT) hipLaunchKernelGGL((k_topk_unit<DD, SC, TT>), grid, block, 0, st, a)
#define LCDA_UNIT(DD)                                                                                      \
    do {                                                                                                   \
        if (kind == 1) LCDA_UNIT3(DD, false, float);                                                      \
        else if (kind == 2) LCDA_UNIT3(DD, false, uint16_t);                                              \
        else if (sc) LCDA_UNIT3(DD, true, void);                                                          \
        else LCDA_UNIT3(DD, false, void);                                                                 \
    } while (0)
    switch (D) {
        case 1: LCDA_UNIT(1); break;
        case 2: LCDA_UNIT(2); break;
        case 4: LCDA_UNIT(4); break;
        default: LCDA_UNIT(8); break;
    }
#undef LCDA_UNIT
#undef LCDA_UNIT3
    return hipGetLastError();
}

}  // namespace lcda
