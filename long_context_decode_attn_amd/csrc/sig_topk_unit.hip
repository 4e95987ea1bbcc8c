// sig_topk_unit.hip - HashAttention SCORE + TOPK over 32-bit signatures in one
// launch: the distances are computed once and kept in LDS, and the workgroups
// that share a (batch item, KV head) exchange their histograms.
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
// Work unit: one (b, KV head) with its G <= 4 query heads, whose n positions
// are cut into Q parts of P positions; one workgroup of 16 wavefronts per
// part, all of a launch resident at once (the host launches this kernel only
// when the grid fits the device one workgroup per CU).
//   1. The part's codes are read once (each load instruction of a wavefront
//      covers 1 KB of consecutive codes) and every (position, query head)
//      distance goes into a 33-bin histogram (one LDS copy per lane, so that
//      the 64 increments of one instruction fall into distinct banks; two
//      heads share a copy's word as 16-bit counts) and, as one byte, into the
//      part's LDS distance array, head by head.  The sink and recent window portions of the part get histograms
//      of their own.
//   2. Every workgroup publishes its three histograms per head, as cumulative
//      counts (C[d] = positions with distance below d), with device-scope stores and arrives at the unit's counter; the last to
//      arrive releases the others by advancing the unit's epoch word.  A
//      workgroup that waits too long (its partners not resident) computes the
//      missing histograms from the codes itself, so the result never depends
//      on co-residency.
//   3. One wavefront per query head reads every part's histograms (lane =
//      part): t and the quota, the ties before this part, and every part's
//      output count (its positions below t, the ties it takes - the lowest
//      ones first - and its window positions outside the top m), hence this
//      part's output offset.
//   4. Each thread owns 4 D consecutive positions of the part and compares
//      their distance bytes, four at a time, with t and t + 1 (byte-parallel
//      subtraction: every byte is below 128, so the sign bit of byte j of
//      (d | 0x80) - t says whether d_j >= t); a dot product with 1, 2, 4, 8
//      turns four sign bits into a nibble of the thread's position masks.  A
//      workgroup scan of the tie counts gives each thread the ties it takes, a
//      second of the selected counts its output offset; it stores its
//      positions in order.
// With the rows of the cache (sparse_decode_step) the same workgroups then run
// GATHER-ATT ("HashAttention ...", slide "Only selection is approximate;
// selected KV stay in full form": attention renormalised over the selected
// rows, read straight from the cache by position):
//   5. each part's selected positions of every head also go into an LDS list
//      (as offsets in the part); 16 / G wavefronts per query head walk the
//      head's list, four rows per load instruction (16 lanes per row, 8 values
//      per lane), with an online softmax in base 2, and merge into one partial
//      state (m, l, acc) per head and part;
//   6. the last workgroup of the unit to publish its partial states merges the
//      parts exactly through their maxima (the split identity of the dense path).
// The workspace holds the counters, epochs and histograms; the counter word is
// (tag << 32 | arrivals) as for the split pass (see arrive_count), so no call
// needs it cleared, and every call leaves it at (tag, 0).

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "sig_proj.h"

namespace lcda {
namespace {

constexpr int kUT = 1024;                       // threads per workgroup
constexpr int kUW = kUT / 64;                   // wavefronts
constexpr int kUBins = 33;
constexpr int kURow = 36;                       // words per published histogram row (34 cumulative counts)
constexpr uint32_t kHi = 0x80808080u;
constexpr uint32_t kPadDist = 0x7Fu;            // distance byte of a position past the end: never < t, never t

template <int D>
struct __align__(16) UnitSmem {
    uint32_t dist[4][kUT * D];                  // [head][dword]: the part's distances, a byte per position
    uint32_t cnt[2 * (kUBins + 1) * 64];        // [head pair][bin][lane]: heads 2p, 2p + 1 in the low and high
                                                // 16 bits; bin 33 takes positions past the end
    uint32_t win[2][4][kUBins];                 // the part's sink and recent window portions
    uint32_t s_w[2][kUW];                       // block scans
    int s_sel[4][4];                            // per head: t, quota, ties before the part, output offset
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

// Exclusive prefixes of x0 and x1 over the workgroup's threads in order, and
// their totals.  Ends with a barrier after its last LDS read.
__device__ __forceinline__ void block_scan2(uint32_t x0, uint32_t x1, uint32_t (*s_w)[kUW], uint32_t& e0,
                                            uint32_t& e1, uint32_t& t0, uint32_t& t1) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t i0 = scan_incl(x0), i1 = scan_incl(x1);
    if (lane == 63) {
        s_w[0][w] = i0;
        s_w[1][w] = i1;
    }
    __syncthreads();
    uint32_t b0 = 0, b1 = 0, a0 = 0, a1 = 0;
#pragma unroll
    for (int k = 0; k < kUW; ++k) {
        const uint32_t v0 = s_w[0][k], v1 = s_w[1][k];
        b0 += k < w ? v0 : 0u;
        b1 += k < w ? v1 : 0u;
        a0 += v0;
        a1 += v1;
    }
    __syncthreads();
    e0 = b0 + i0 - x0;
    e1 = b1 + i1 - x1;
    t0 = a0;
    t1 = a1;
}

// Dword dw (positions 4 dw .. 4 dw + 3) of a head's distance array: thread T of
// the compaction owns dwords D T .. D T + D - 1.  With D = 8 (two 16-byte
// chunks per thread) the chunks of a thread are swapped for odd T / 8, so that
// 16 neighbouring threads' reads of one chunk each fall into distinct banks.
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

// The four sign bits of a dword of distance bytes as a nibble.
__device__ __forceinline__ uint32_t nibble(uint32_t s) { return __builtin_amdgcn_udot4(s >> 7, 0x08040201u, 0u, false); }

// Histograms of the positions [beg, end) of a unit for heads g < G, counted
// into the LDS copies (which the caller has zeroed) and, for the positions in
// the windows, into win; reads the codes from memory.  The fallback of a
// workgroup whose partners did not arrive in time.
template <int D>
__device__ void count_part(const TopkArgs& a, UnitSmem<D>& sm, const uint32_t* ks, const uint32_t (&q)[4], int beg,
                           int end, int s_end, int r_beg) {
    const int lane = threadIdx.x & 63;
    for (int i = beg + (int)threadIdx.x; i < end; i += kUT) {
        const uint32_t x = ks[i];
        const int pt = i < s_end ? 0 : (i >= r_beg ? 1 : -1);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if (g < a.G) {
                const uint32_t d = (uint32_t)__builtin_popcount(x ^ q[g]);
                __hip_atomic_fetch_add(&sm.cnt[(((g >> 1) * (kUBins + 1) + d) << 6) + lane], 1u << (16 * (g & 1)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (pt >= 0)
                    __hip_atomic_fetch_add(&sm.win[pt][g][d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
}

// Publish the part's histograms as cumulative counts: row (kind, head) of
// prow = [part, sink, recent][head][kURow] gets C[d], d = 0 .. 33, the number
// of the kind's positions with distance below d.  Wavefront 4 kind + head
// (lane = bin) sums the bin over the lane copies and scans over the bins.
template <int D>
__device__ __forceinline__ void publish(const TopkArgs& a, const UnitSmem<D>& sm, uint32_t* prow) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (w >= 12) return;
    const int kind = w >> 2, g = w & 3;
    uint32_t v = 0;
    if (g < a.G && lane < kUBins) {
        if (kind == 0) {
            const uint32_t* r = sm.cnt + (((g >> 1) * (kUBins + 1) + lane) << 6);
            const int sh = 16 * (g & 1);
#pragma unroll 8
            for (int c = 0; c < 64; ++c) v += (r[(c + lane) & 63] >> sh) & 0xFFFFu;   // lane-rotated: distinct banks
        } else {
            v = sm.win[kind - 1][g][lane];
        }
    }
    const uint32_t incl = scan_incl(v);
    uint32_t* row = prow + (kind * 4 + g) * kURow;
    if (lane < kUBins) store_dev(row + lane + 1, incl);
    if (lane == 0) store_dev(row, 0u);
}

template <int D>
__device__ __forceinline__ void zero_counts(UnitSmem<D>& sm) {
    for (int k = threadIdx.x; k < 2 * (kUBins + 1) * 64; k += kUT) sm.cnt[k] = 0u;
    for (int k = threadIdx.x; k < 2 * 4 * kUBins; k += kUT) (&sm.win[0][0][0])[k] = 0u;
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

// GATHER-ATT over this part's selected positions of each query head, then the
// merge of the parts (see the file comment, steps 5 and 6).
template <typename T, int D>
__device__ void gather_part(const TopkArgs& a, UnitSmem<D>& sm, const uint16_t* lst, bool in_lds, const int (&cntg)[4],
                            const int (&lbase)[4], int unit, int part, int64_t row0, int b, int h, int pbeg) {
    constexpr int U = sizeof(T) == 2 ? 4 : 2;   // rows per lane group and step (fewer for fp32 rows)
    constexpr int kStep = 4 * U;         // rows per wavefront and step
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
        const int cnt = __builtin_amdgcn_readfirstlane(gw == 0 ? cntg[0] : gw == 1 ? cntg[1] : gw == 2 ? cntg[2] : cntg[3]);
        const int lb = __builtin_amdgcn_readfirstlane(gw == 0 ? lbase[0] : gw == 1 ? lbase[1] : gw == 2 ? lbase[2] : lbase[3]);
        const int64_t head = (a.kv_batch_stride == 0 ? 0 : (int64_t)b * a.kv_batch_stride) + (int64_t)h * a.n * kD;
        const T* kh = static_cast<const T*>(a.gk) + head + 8 * c16;
        const T* vh = static_cast<const T*>(a.gv) + head + 8 * c16;
        const int32_t* ilist = a.idx + row * a.cap + sm.s_sel[gw][3];   // the part's entries of the index list
        float qv[8];
        {
            GRow<T> x;
            x.load(static_cast<const T*>(a.gq) + row * kD + 8 * c16);
            x.to_float(qv);
        }
        struct Step {
            GRow<T> k[U], v[U];
        };
        // The rows of entries t0 + 4 u + j of the part's list (clamped to the
        // last entry; rows past cnt are masked in compute).  LISTED: the
        // positions come from the LDS list; otherwise from the index list the
        // workgroup has written (a list too long for LDS).
        auto fetch = [&](Step& st, int t0, auto listed) {
            int pos[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = min(t0 + 4 * u + j, cnt - 1);
                if constexpr (decltype(listed)::value) pos[u] = pbeg + (int)lst[lb + t];
                else pos[u] = (int)load_dev_u32(reinterpret_cast<const uint32_t*>(ilist) + t);
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
    if (w < G) {
        PartMerge pm{Q, a.pml, a.pacc, nullptr, nullptr, a.out, a.alpha};
        combine_row(pm, row0 + w, lane);
    }
}

// D: dwords per thread and head; a part holds P = 4096 D positions.  T: the
// rows' type for the fused GATHER-ATT (float or uint16_t for bf16), void for
// TOPK alone.
template <int D, bool SCORES, typename T>
__global__ __launch_bounds__(kUT) void k_topk_unit(TopkArgs a) {
    constexpr int P = 4 * kUT * D;
    __shared__ UnitSmem<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int Q = a.parts;
    // Workgroup -> (unit, part): part-major, so that with a multiple of 8 units
    // the parts of a unit run on one XCD (workgroups go round the 8 XCDs in
    // turn) and every XCD holds every part position equally.
    const int units = a.B * a.Hkv;
    const int unit = blockIdx.x % units, part = blockIdx.x / units;
    const int b = unit / a.Hkv, h = unit % a.Hkv;
    const int G = a.G;
    const int n = (int)a.n;
    const int pbeg = part * P, pend = min(n, pbeg + P);
    const uint32_t* ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n;
    const int64_t row0 = (int64_t)b * a.Hq + (int64_t)h * G;
    const int s_end = (int)min(a.n_sink, a.n);
    const int r_beg = (int)max((int64_t)s_end, a.n - a.n_recent);
    const bool vec = (n & 3) == 0;   // uniform

    // ---- 1. distances ------------------------------------------------------------------
    // The query codes first (so that waiting for them is not waiting for all the
    // codes), then step s: positions pbeg + 4 (1024 s + tid) + e, e < 4; every
    // step's codes are requested at once.
    uint32_t q[4];
    if (a.q == nullptr) {
#pragma unroll
        for (int g = 0; g < 4; ++g) q[g] = a.q_sigs[row0 + min(g, G - 1)];
    }
    u32x4 xc[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        const int i = pbeg + 4 * (kUT * s + tid);
        if (vec) {
            xc[s] = ld16(ks + min(i, n - 4));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) xc[s][e] = ks[min(i + e, n - 1)];
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
    __syncthreads();

    uint32_t* mycnt = sm.cnt + lane;
#pragma unroll
    for (int s = 0; s < D; ++s) {
        const int i = pbeg + 4 * (kUT * s + tid);
        const int dw = dist_slot<D>(kUT * s + tid);
        if (pbeg + 4 * kUT * (s + 1) <= n) {   // uniform: every position of the step is below n
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g < G) {   // uniform
                    uint32_t pk = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t d = (uint32_t)__builtin_popcount(xc[s][e] ^ q[g]);
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
                    uint32_t pk = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = i + e < n;
                        const uint32_t d = ok ? (uint32_t)__builtin_popcount(xc[s][e] ^ q[g]) : (uint32_t)kUBins;
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
    // Window portions of the part, from the distance bytes.
    {
        const int wb0 = pbeg, we0 = min(pend, s_end);           // sink portion [wb0, we0)
        const int wb1 = max(pbeg, r_beg), we1 = pend;          // recent portion [wb1, we1)
        for (int k = tid; k < max(we0 - wb0, 0) + max(we1 - wb1, 0); k += kUT) {
            const int pt = k < max(we0 - wb0, 0) ? 0 : 1;
            const int i = pt == 0 ? wb0 + k : wb1 + (k - max(we0 - wb0, 0));
            const int r = i - pbeg;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (g < G) {
                    const uint32_t d = (sm.dist[g][dist_slot<D>(r >> 2)] >> (8 * (r & 3))) & 0xFFu;
                    __hip_atomic_fetch_add(&sm.win[pt][g][d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. exchange --------------------------------------------------------------------------
    uint32_t* phist = a.phist + (int64_t)unit * Q * 3 * 4 * kURow;
    publish(a, sm, phist + (int64_t)part * 3 * 4 * kURow);
    wait_vm_all();      // this thread's histogram stores are acknowledged
    __syncthreads();    // ... in every thread
    if (Q > 1) {
        if (tid == 0) {
            uint32_t* ep = a.epoch + unit;
            const uint32_t e = __hip_atomic_load(ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_vm_all();  // the epoch is read before this workgroup arrives
            unsigned long long* c = a.bar + unit;
            const uint32_t tag = ctr_tag(c);
            const unsigned long long valid0 = (unsigned long long)tag << 32;
            unsigned long long old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t count;
            if ((uint32_t)(old >> 32) == tag) {
                count = (uint32_t)old + 1u;
            } else {   // a word this library did not leave: install (tag, 1) or count on the installed word
                unsigned long long cur = old + 1ull;
                while (true) {
                    if ((uint32_t)(cur >> 32) == tag) {
                        old = __hip_atomic_fetch_add(c, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        count = (uint32_t)old + 1u;
                        break;
                    }
                    if (__hip_atomic_compare_exchange_strong(c, &cur, valid0 | 1ull, __ATOMIC_RELAXED,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                        count = 1u;
                        break;
                    }
                }
            }
            int released = 0;
            if (count == (uint32_t)Q) {   // the last to arrive: reset the counter, then release the others
                __hip_atomic_store(c, valid0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ep, e + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                released = 1;
            } else {
                for (int it = 0; it < a.spin_max; ++it) {
                    if (__hip_atomic_load(ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != e) {
                        released = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            sm.s_flag = released;
        }
        __syncthreads();
        if (!sm.s_flag) {   // uniform: the partners did not arrive in time; count their parts here
            for (int p = 0; p < Q; ++p) {
                if (p == part) continue;
                zero_counts(sm);
                __syncthreads();
                count_part(a, sm, ks, q, p * P, min(n, p * P + P), s_end, r_beg);
                __syncthreads();
                publish(a, sm, phist + (int64_t)p * 3 * 4 * kURow);
                __syncthreads();
            }
            wait_vm_all();
            __syncthreads();
        }
    }

    // ---- 3. selection: one wavefront per query head ------------------------------------------
    // Row (p, kind, g) of phist: C_p[d], d = 0 .. 33.
    auto crow = [&](int p, int kind, int g) { return phist + (((int64_t)p * 3 + kind) * 4 + g) * kURow; };
    if (w < G) {
        const int g = w;
        // Lane d: S[d] = positions of the unit with distance <= d; the requests
        // of up to 8 parts are issued together.
        uint32_t S = 0;
        if (lane < kUBins) {
            for (int p0 = 0; p0 < Q; p0 += 8) {
                uint32_t v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = p0 + k < Q ? load_dev_u32(crow(p0 + k, 0, g) + lane + 1) : 0u;
#pragma unroll
                for (int k = 0; k < 8; ++k) S += v[k];
            }
        }
        const uint32_t meff = (uint32_t)min(a.m, a.n);
        const uint64_t reach = __ballot(lane < kUBins && meff > 0 && S >= meff);
        const int t = reach ? (int)__builtin_ctzll(reach) : -1;
        const uint32_t below_all = t > 0 ? lane_val(S, t - 1) : 0u;
        const uint32_t quota = t >= 0 ? meff - below_all : 0u;
        // Lane p (a part): positions below t, ties, and the same for its window
        // portions, from C_p[t] and C_p[t + 1] of each kind.
        const int qb = lane * P, qe = min(n, qb + P);
        const bool part_ok = lane < Q && t >= 0;
        const bool in_s = part_ok && qb < s_end, in_r = part_ok && qe > r_beg;
        const int tt = t >= 0 ? t : 0;
        uint32_t c0 = 0, c1 = 0, s0 = 0, s1 = 0, r0 = 0, r1 = 0;
        if (part_ok) {
            c0 = load_dev_u32(crow(lane, 0, g) + tt);
            c1 = load_dev_u32(crow(lane, 0, g) + tt + 1);
        }
        if (in_s) {
            s0 = load_dev_u32(crow(lane, 1, g) + tt);
            s1 = load_dev_u32(crow(lane, 1, g) + tt + 1);
        }
        if (in_r) {
            r0 = load_dev_u32(crow(lane, 2, g) + tt);
            r1 = load_dev_u32(crow(lane, 2, g) + tt + 1);
        }
        const uint32_t below = c0, ties = c1 - c0, ws_t = s1 - s0, wr_t = r1 - r0;
        const uint32_t ties_before = scan_incl(ties) - ties;
        const uint32_t taken = quota > ties_before ? min(quota - ties_before, ties) : 0u;
        // The ties a part takes are its lowest ones: the sink portion (a prefix
        // of the part) takes the first of them, the recent portion (a suffix)
        // what is left after the ties before it.
        const uint32_t tk_s = min(ws_t, taken);
        const uint32_t tk_r = taken > ties - wr_t ? min(taken - (ties - wr_t), wr_t) : 0u;
        const uint32_t win_n = (uint32_t)(max(min(qe, s_end) - qb, 0) + max(qe - max(qb, r_beg), 0));
        const uint32_t cnt = lane < Q ? below + taken + win_n - (s0 + tk_s + r0 + tk_r) : 0u;
        const uint32_t cincl = scan_incl(cnt);
        // Every lane takes part in the reads (readlane outside divergent code).
        const uint32_t my_tb = lane_val(ties_before, part);
        const uint32_t my_off = lane_val(cincl, part) - lane_val(cnt, part);
        const uint32_t total = lane_val(cincl, 63);
        if (lane == 0) {
            sm.s_sel[g][0] = t;
            sm.s_sel[g][1] = (int)quota;
            sm.s_sel[g][2] = (int)my_tb;
            sm.s_sel[g][3] = (int)my_off;
            sm.s_total[g] = (int)total;
        }
    }
    __syncthreads();

    // ---- 4. ordered compaction -----------------------------------------------------------------
    // Thread tid: positions P0 .. P0 + 4 D - 1 of the part (bit j of its masks).
    const int P0 = pbeg + 4 * D * tid;
    uint32_t lt[4], eq[4], tiesv[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        lt[g] = eq[g] = tiesv[g] = 0u;
        if (g < G) {
            const int t = sm.s_sel[g][0];
            const uint32_t T0 = t >= 0 ? (uint32_t)t * 0x01010101u : 0u;   // t = -1 (m = 0): nothing below
            const uint32_t T1 = t >= 0 ? (uint32_t)(t + 1) * 0x01010101u : 0u;
            uint32_t l = 0, le = 0;
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const uint32_t A = sm.dist[g][dist_slot<D>(D * tid + j)] | kHi;
                l |= nibble(~(A - T0) & kHi) << (4 * j);
                le |= nibble(~(A - T1) & kHi) << (4 * j);
            }
            lt[g] = l;
            eq[g] = le & ~l;
            tiesv[g] = __builtin_popcount(eq[g]);
        }
    }
    uint32_t te01, te23, tt01, tt23;
    block_scan2(tiesv[0] | (tiesv[1] << 16), tiesv[2] | (tiesv[3] << 16), sm.s_w, te01, te23, tt01, tt23);
    const uint32_t winm = (low_bits(s_end - P0) | ~low_bits(r_beg - P0)) & low_bits(n - P0) & low_bits(4 * D);
    uint32_t sel[4], nsel[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        sel[g] = nsel[g] = 0u;
        if (g < G) {
            const uint32_t local = ((g < 2 ? te01 : te23) >> (16 * (g & 1))) & 0xFFFFu;
            const uint32_t before = (uint32_t)sm.s_sel[g][2] + local;
            const uint32_t quota = (uint32_t)sm.s_sel[g][1];
            const uint32_t take = quota > before ? min(quota - before, tiesv[g]) : 0u;
            uint32_t tk = 0;
            if (take == tiesv[g]) {
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
    uint32_t oe01, oe23, ot01, ot23;
    block_scan2(nsel[0] | (nsel[1] << 16), nsel[2] | (nsel[3] << 16), sm.s_w, oe01, oe23, ot01, ot23);
    // The part's selected positions of head g: cntg[g] of them, listed in LDS
    // (offsets from pbeg, after the lists of the heads before) when they fit.
    constexpr bool kGather = !std::is_void<T>::value;
    int cntg[4], lbase[4];
    int lsum = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        cntg[g] = g < G ? (int)(((g < 2 ? ot01 : ot23) >> (16 * (g & 1))) & 0xFFFFu) : 0;
        lbase[g] = lsum;
        lsum += cntg[g];
    }
    uint16_t* lst = reinterpret_cast<uint16_t*>(&sm.dist[0][0]);
    const bool in_lds = kGather && lsum <= (int)(sizeof(sm.dist) / 2);   // uniform
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
            uint32_t pos4 = 4u * ((uint32_t)sm.s_sel[g][3] + local);
            int li = lbase[g] + (int)local;
            uint32_t s = sel[g];
            while (s) {
                const int bit = __builtin_ctz(s);
                __builtin_amdgcn_raw_buffer_store_b32(P0 + bit, ro, pos4, 0, 0);
                if (in_lds) lst[li++] = (uint16_t)(P0 + bit - pbeg);
                pos4 += 4u;
                s &= s - 1u;
            }
            if (part == 0) {
                if (tid == 0) a.count[row0 + g] = total;
                for (int64_t i = (int64_t)total + tid; i < a.cap; i += kUT) out[i] = -1;
            }
        }
    }
    if constexpr (kGather) {
        wait_vm_all();      // the index stores are acknowledged (a list too long for LDS is read back)
        __syncthreads();
        gather_part<T>(a, sm, lst, in_lds, cntg, lbase, unit, part, row0, b, h, pbeg);
    }
}

}  // namespace

// Positions per part for a unit of n positions when `units` units share the
// device's `cus` compute units: parts of 4096 D positions (D = 1, 2, 4, 8),
// the smallest D with units * parts <= cus; 0 when none fits or G > 4.
int topk_unit_part(int64_t n, int units, int G, int cus) {
    if (n <= 0 || G > 4 || units <= 0) return 0;
    for (int D = 1; D <= 8; D *= 2) {
        const int64_t P = 4096 * (int64_t)D;
        const int64_t parts = (n + P - 1) / P;
        if (parts <= 64 && (int64_t)units * parts <= cus) return (int)P;
    }
    return 0;
}

int topk_unit_row_words() { return kURow; }

hipError_t launch_topk_unit(const TopkArgs& a, int dtype, hipStream_t st) {
    const int D = a.part_len / 4096;
    if (a.B <= 0 || a.G > 4 || a.parts <= 0 || a.part_len != 4096 * D || (D != 1 && D != 2 && D != 4 && D != 8))
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
