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
// Three launches; each head's positions are cut into chunks of L positions.
//   1. k_wide_hist, one workgroup per (chunk, KV head, group of up to 8 query
//      heads): reads the chunk's key codes once for the whole group (two
//      batches of loads in flight: the next batch loads while the current one
//      is counted), counts each head's (b + 1)-bin distance histogram of the
//      chunk in LDS (several lane copies, so that lanes with equal distances
//      rarely meet on one word), and, for W >= 2, keeps the distances as bytes
//      (min(d, 255)), the group's bytes of a position side by side, so one
//      store per position writes them.  Chunks that meet the sink or the
//      recent window also count the histogram of their window positions alone.
//   2. k_wide_select, one workgroup of 1,024 threads per query head: the
//      threshold t (first bin whose prefix over the summed histograms reaches
//      m) and the quota of ties at t the top m takes; then, per chunk, the ties
//      at t before it and the positions selected before it, both from
//      histogram sums: a window's part of a chunk is a prefix (sink) or a
//      suffix (recent) of the chunk, so its ties are the chunk's first (last)
//      ties and their ranks are known.  Up to 32 chunks' histograms of all
//      three kinds are staged in LDS with one round of 16-byte loads.
//   3. k_wide_compact, one workgroup per (chunk, KV head, group): ordered
//      compaction of the chunk in tiles of 4,096 positions (16 consecutive per
//      thread), one block scan of the tie counts and one of the selection
//      counts per tile, two heads packed per scanned word.  For W = 1 the
//      distances are computed again from the codes (as cheap to read as the
//      bytes); for W >= 2 they come from the stored bytes (four heads' bytes
//      compared with their thresholds at once where a group has four or
//      eight heads), and a byte of 255 is resolved from the codes when
//      t >= 255.
// No workgroup waits for another: the launches order the passes.

#include "common.h"
#include "internal.h"
#include "wide.h"

namespace lcda {
namespace {

constexpr int kWT = 256;                         // threads per workgroup, histogram and compaction passes
constexpr int kST = 1024;                        // threads per workgroup, select pass
constexpr int kPT = 16;                          // compaction: positions per thread and tile
constexpr int kTile = kWT * kPT;
constexpr int kMaxBins = 32 * 16 + 1;
constexpr int kMaxBinsP = (kMaxBins + 7) / 8 * 8;   // histogram rows padded to 16 bytes
constexpr int kSelCB = 32;                       // chunks per block in the select pass

constexpr int pow2_floor(int x) { return x >= 16 ? 16 : x >= 8 ? 8 : x >= 4 ? 4 : x >= 2 ? 2 : 1; }

template <int W, int HG>
struct WideCfg {
    static constexpr int kBins = 32 * W + 1;
    static constexpr int kBinsP = (kBins + 7) / 8 * 8;
    // lane copies of the group's histogram: about 24 KB of LDS at most
    static constexpr int kCopies = pow2_floor(6144 / (HG * kBins));
    static constexpr int kStride = (HG * kBins) | 1;       // words per copy (odd: copies of a bin in distinct banks)
    static constexpr int kPP = W >= 4 ? 1 : 4 / W;         // positions per item (one item = max(W, 4) words)
    static constexpr int kItemWords = kPP * W;
    static constexpr bool kStore = W >= 2;                 // distances kept as bytes
    static constexpr int kU = W >= 4 ? 2 : 1;              // items per thread and batch
    static constexpr int kGranule = 2 * kWT * kU * kPP;   // positions of one turn of the loop
    // wavefronts per SIMD the register budget is set for (8: at most 64 VGPRs)
    static constexpr int kHistWaves = W >= 2 && W <= 8 && HG <= 4 ? 8 : 4;
    static constexpr int kCompactWaves = kStore && HG <= 4 ? 7 : 2;
};

__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// The (b, KV head, head group) a workgroup works on, from its unit index.
struct WideUnit {
    int64_t row0;           // first query row (b * Hq + hq) of the group
    int GH;                 // heads in the group
    const uint32_t* ks;     // the KV head's codes, [n][W]
    uint8_t* dist;          // the group's distance bytes, [n][HG]
};
template <int HG>
__device__ __forceinline__ WideUnit wide_unit(const WideArgs& a, int unit) {
    const int grp = unit % a.ng, bh = unit / a.ng;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    WideUnit u;
    u.row0 = (int64_t)b * a.Hq + (int64_t)h * a.G + grp * HG;
    u.GH = min(HG, a.G - grp * HG);
    u.ks = a.key_sigs + ((int64_t)b * a.Hkv + h) * a.n * a.W;
    u.dist = a.dist + (int64_t)unit * a.dstride;
    return u;
}

// Offset of the histogram row (kind slot, query row, chunk c); rows of binsP u16.
__device__ __forceinline__ int64_t hist_at(const WideArgs& a, int slot, int64_t row, int64_t c, int binsP) {
    return ((slot * ((int64_t)a.B * a.Hq) + row) * a.nc + c) * binsP;
}

// Words [w0, w0 + NW) of the codes, vector loads where aligned and inside the
// codes, else word loads with clamped addresses (entries past the end unused).
template <int NW>
__device__ __forceinline__ void load_words(uint32_t (&x)[NW], const uint32_t* ks, int64_t w0, int64_t nW, bool vec) {
    if (NW % 4 == 0 && vec && w0 + NW <= nW) {
#pragma unroll
        for (int v = 0; v < NW / 4; ++v) {
            const u32x4 y = ld16(ks + w0 + 4 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * v + e] = y[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < NW; ++e) x[e] = ks[min(w0 + e, nW - 1)];
    }
}

template <int W>
__device__ __forceinline__ uint32_t distance(const uint32_t* x, const uint32_t* q) {
    uint32_t d = 0;
#pragma unroll
    for (int k = 0; k < W; ++k) d += (uint32_t)__builtin_popcount(x[k] ^ q[k]);
    return d;
}

// ---- 1. distances and histograms ----------------------------------------------
// One chunk of one head group.  Offsets are 32-bit from the chunk's first
// position (a chunk holds at most kWideMaxL positions).  VEC: the codes are
// read as aligned 16-byte vectors (every item lies inside the codes); else
// word by word, clamped into the chunk.
template <int W, int HG, bool VEC>
struct HistPass {
    using C = WideCfg<W, HG>;
    const WideArgs& a;
    const WideUnit& u;
    uint32_t (&q)[HG][W];
    uint32_t* hist = nullptr;        // the histogram copies, then one spare word per lane
    int my = 0;                      // this lane's copy: its first word
    int spare = 0;                   // this lane's spare word
    const uint32_t* kc = nullptr;    // codes of the chunk's first position
    uint8_t* dc = nullptr;           // distance bytes of the chunk's first position
    int64_t p0 = 0;                  // the chunk's first position
    int len = 0, items = 0, tid = 0;

    // Every lane loads (items past the end repeat the last item), computes
    // every distance and makes every atomic: a position past the end (or a
    // head past a partial group) counts into the lane's spare LDS word (its
    // own, so that such lanes do not meet on one word), and a repeated item
    // stores its own bytes again, at its own positions.  With no branch around
    // a load's use, the compiler's wait for one batch never covers the batch
    // loaded after it.
    __device__ __forceinline__ void load(uint32_t (&x)[C::kU][C::kItemWords], int i0) const {
#pragma unroll
        for (int v = 0; v < C::kU; ++v) {
            const int it = min(i0 + v * kWT + tid, items - 1);
            const uint32_t* src = kc + it * C::kItemWords;
            if constexpr (VEC) {
#pragma unroll
                for (int k = 0; k < C::kItemWords / 4; ++k) {
                    const u32x4 y = ld16(src + 4 * k);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[v][4 * k + e] = y[e];
                }
            } else {
                const int last = len * W - 1 - it * C::kItemWords;
#pragma unroll
                for (int e = 0; e < C::kItemWords; ++e) x[v][e] = src[min(e, last)];
            }
        }
    }
    __device__ __forceinline__ void count(const uint32_t (&x)[C::kU][C::kItemWords], int i0) const {
#pragma unroll
        for (int v = 0; v < C::kU; ++v) {
            const int it = i0 + v * kWT + tid;
#pragma unroll
            for (int e = 0; e < C::kPP; ++e) {
                const int p = it * C::kPP + e;
                const bool ok = p < len;
                uint32_t packed[(HG + 3) / 4] = {};
#pragma unroll
                for (int j = 0; j < HG; ++j) {
                    const uint32_t d = distance<W>(&x[v][e * W], q[j]);
                    const int at = ok && j < u.GH ? my + j * C::kBins + (int)d : spare;
                    __hip_atomic_fetch_add(&hist[at], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    packed[j / 4] |= min(d, 255u) << (8 * (j % 4));
                    if (a.scores && ok && j < u.GH) a.scores[(u.row0 + j) * a.n + p0 + p] = (int16_t)(-(int)d);
                }
                // the position the lane's codes belong to (a repeated item's own); past the end, no store
                const int pc = min(it, items - 1) * C::kPP + e;
                if (C::kStore && pc < len) {
                    uint8_t* dp = dc + pc * HG;
                    if constexpr (HG == 1) *dp = (uint8_t)packed[0];
                    else if constexpr (HG == 2) *reinterpret_cast<uint16_t*>(dp) = (uint16_t)packed[0];
                    else if constexpr (HG == 4) *reinterpret_cast<uint32_t*>(dp) = packed[0];
                    else *reinterpret_cast<uint2*>(dp) = make_uint2(packed[0], packed[1]);
                }
            }
        }
    }
};

template <int W, int HG, bool VEC>
__global__ __launch_bounds__(kWT, (WideCfg<W, HG>::kHistWaves)) void k_wide_hist(WideArgs a) {
    using C = WideCfg<W, HG>;
    __shared__ uint32_t hist[C::kCopies * C::kStride + 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t c = (int64_t)blockIdx.x % a.nc;
    const WideUnit u = wide_unit<HG>(a, (int)((int64_t)blockIdx.x / a.nc));
    const int64_t n = a.n;
    uint32_t q[HG][W];
#pragma unroll
    for (int j = 0; j < HG; ++j)
#pragma unroll
        for (int k = 0; k < W; ++k) q[j][k] = a.q_sigs[(u.row0 + min(j, u.GH - 1)) * W + k];
    for (int k = tid; k < C::kCopies * C::kStride; k += kWT) hist[k] = 0u;
    __syncthreads();

    HistPass<W, HG, VEC> hp{a, u, q};
    hp.hist = hist;
    hp.my = (lane % C::kCopies) * C::kStride;
    hp.spare = C::kCopies * C::kStride + lane;
    hp.p0 = c * a.L;
    hp.kc = u.ks + hp.p0 * W;
    hp.dc = u.dist + hp.p0 * HG;
    hp.len = (int)(min(n, hp.p0 + a.L) - hp.p0);
    hp.items = (hp.len + C::kPP - 1) / C::kPP;
    hp.tid = tid;
    constexpr int kStep = kWT * C::kU;
    // two batches in flight: B loads while A is counted, then A while B is;
    // both load on every turn (past the end they repeat the last item, which
    // then counts into the spare word), so no branch joins paths with
    // different loads outstanding
    uint32_t xa[C::kU][C::kItemWords], xb[C::kU][C::kItemWords];
    hp.load(xa, 0);
    for (int i0 = 0; i0 < hp.items; i0 += 2 * kStep) {
        hp.load(xb, i0 + kStep);
        hp.count(xa, i0);
        hp.load(xa, i0 + 2 * kStep);
        hp.count(xb, i0 + kStep);
    }
    __syncthreads();
    for (int k = tid; k < u.GH * C::kBins; k += kWT) {
        uint32_t s = 0;
#pragma unroll
        for (int cp = 0; cp < C::kCopies; ++cp) s += hist[cp * C::kStride + k];
        const int j = k / C::kBins, bin = k % C::kBins;
        a.hist[hist_at(a, 0, u.row0 + j, c, C::kBinsP) + bin] = (uint16_t)s;
    }

    // Window parts of the chunk (only when the windows are disjoint; when they
    // meet, every position is selected and the selection needs no counts).
    const int64_t s_end = min(a.n_sink, n), r_beg = max((int64_t)0, n - a.n_recent);
    if (s_end >= r_beg) return;
    const int64_t p1 = hp.p0 + hp.len;
#pragma unroll 1
    for (int slot = 1; slot <= 2; ++slot) {
        const int64_t q0 = slot == 1 ? hp.p0 : max(hp.p0, r_beg);
        const int64_t q1 = slot == 1 ? min(p1, s_end) : p1;
        if (q0 >= q1) continue;   // uniform
        __syncthreads();
        for (int k = tid; k < u.GH * C::kBins; k += kWT) hist[k] = 0u;
        __syncthreads();
        for (int64_t pos = q0 + tid; pos < q1; pos += kWT) {
            uint32_t x[W];
            load_words<W>(x, u.ks, pos * W, n * W, VEC);
#pragma unroll
            for (int j = 0; j < HG; ++j) {
                if (j >= u.GH) continue;
                __hip_atomic_fetch_add(&hist[j * C::kBins + distance<W>(x, q[j])], 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        __syncthreads();
        for (int k = tid; k < u.GH * C::kBins; k += kWT) {
            const int j = k / C::kBins, bin = k % C::kBins;
            a.hist[hist_at(a, slot, u.row0 + j, c, C::kBinsP) + bin] = (uint16_t)hist[k];
        }
    }
}

// ---- 2. threshold, quota and per-chunk offsets -----------------------------------
__global__ __launch_bounds__(kST) void k_wide_select(WideArgs a) {
    __shared__ __align__(16) uint16_t blk[3][kSelCB * kMaxBinsP];
    __shared__ uint32_t tot[kMaxBins];
    __shared__ uint32_t cnt[6][kSelCB];   // below, ties at t: all positions, sink part, recent part
    __shared__ int s_t;
    __shared__ uint32_t s_quota, s_total;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t row = blockIdx.x;
    const int bins = 32 * a.W + 1, binsP = (bins + 7) / 8 * 8;
    const int64_t n = a.n, nc = a.nc, L = a.L;
    const int64_t s_end = min(a.n_sink, n), r_beg = max((int64_t)0, n - a.n_recent);
    const bool meet = s_end >= r_beg;

    // Stage chunks [c0, c0 + cb) of the kinds asked for: every load issued before the first LDS store.
    auto stage = [&](int64_t c0, int cb, bool s0, bool s1, bool s2) {
        const int vecs = cb * binsP / 8;
        const bool on[3] = {s0, s1, s2};
        u32x4 r[3][3];
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            if (!on[s]) continue;
            const u32x4* src = reinterpret_cast<const u32x4*>(a.hist + hist_at(a, s, row, c0, binsP));
#pragma unroll
            for (int k = 0; k < 3; ++k)
                if (tid + k * kST < vecs) r[s][k] = src[tid + k * kST];
        }
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            if (!on[s]) continue;
            u32x4* dst = reinterpret_cast<u32x4*>(&blk[s][0]);
#pragma unroll
            for (int k = 0; k < 3; ++k)
                if (tid + k * kST < vecs) dst[tid + k * kST] = r[s][k];
        }
    };
    auto need1 = [&](int64_t c0) { return !meet && c0 * L < s_end; };
    auto need2 = [&](int64_t c0, int cb) { return !meet && min(n, (c0 + cb) * L) > r_beg; };

    // 1. the row's histogram, summed over the chunks (one staging when nc <= kSelCB)
    const bool one = nc <= kSelCB;
    if (tid < kMaxBins) tot[tid] = 0u;
    for (int64_t c0 = 0; c0 < nc; c0 += kSelCB) {
        const int cb = (int)min((int64_t)kSelCB, nc - c0);
        __syncthreads();   // blk free
        stage(c0, cb, true, one && need1(c0), one && need2(c0, cb));
        __syncthreads();
        if (tid < bins) {
            uint32_t s = 0;
            for (int ci = 0; ci < cb; ++ci) s += blk[0][ci * binsP + tid];
            tot[tid] += s;
        }
    }
    __syncthreads();

    // 2. threshold and quota (wavefront 0; lane l owns bins l*per .. l*per + per - 1)
    const uint32_t meff = (uint32_t)min(a.m, n);
    if (w == 0) {
        constexpr int kPer = (kMaxBins + 63) / 64;
        const int per = (bins + 63) / 64;
        uint32_t cc[kPer], sum = 0;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int bin = lane * per + k;
            cc[k] = k < per && bin < bins ? tot[bin] : 0u;
            sum += cc[k];
        }
        const uint32_t incl = wave_scan_incl(sum);
        const uint64_t reach = __ballot(meff > 0 && incl >= meff);
        if (lane == 0 && !reach) {
            s_t = -1;
            s_quota = 0u;
        }
        if (reach && lane == (int)__builtin_ctzll(reach)) {
            uint32_t run = incl - sum;
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                if (k < per && run + cc[k] >= meff) {
                    s_t = lane * per + k;
                    s_quota = meff - run;
                    break;
                }
                run += cc[k];
            }
        }
    }
    __syncthreads();
    const int t = s_t;
    const uint32_t quota = s_quota;

    // 3. per-chunk offsets, in blocks of kSelCB chunks (wavefront 0 carries the running sums)
    uint32_t carry_t = 0, carry_s = 0;
    for (int64_t c0 = 0; c0 < nc; c0 += kSelCB) {
        const int cb = (int)min((int64_t)kSelCB, nc - c0);
        const bool n1 = need1(c0), n2 = need2(c0, cb);
        if (!one) {
            __syncthreads();   // blk free
            stage(c0, cb, true, n1, n2);
            __syncthreads();
        }
        // 32 threads per chunk: strided partial sums of the bins below t, then a reduction over the 32
        const int ci = tid >> 5, part = tid & 31;
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            if ((s == 1 && !n1) || (s == 2 && !n2)) {
                if (tid < kSelCB) cnt[2 * s][tid] = cnt[2 * s + 1][tid] = 0u;
                continue;
            }
            uint32_t below = 0;
            if (ci < cb)
                for (int k = part; k < t; k += 32) below += blk[s][ci * binsP + k];
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) below += __shfl_xor(below, o, 64);
            if (ci < cb && part == 0) {
                cnt[2 * s][ci] = below;
                cnt[2 * s + 1][ci] = t >= 0 ? (uint32_t)blk[s][ci * binsP + t] : 0u;
            }
        }
        __syncthreads();
        if (w == 0) {
            const int64_t c = c0 + lane;
            const bool on = lane < cb;
            const int64_t p0 = c * L, p1 = min(n, p0 + L);
            const uint32_t below = on ? cnt[0][lane] : 0u, ties = on ? cnt[1][lane] : 0u;
            const uint32_t ti = wave_scan_incl(ties);
            const uint32_t tb = carry_t + ti - ties;   // ties at t before the chunk
            uint32_t sel = 0;
            if (on) {
                if (meet) {
                    sel = (uint32_t)(p1 - p0);
                } else {
                    auto take = [&](uint32_t before, uint32_t k) {   // of k ties ranked from `before`, those in the top
                        const int64_t r = (int64_t)quota - (int64_t)before;
                        return (uint32_t)max((int64_t)0, min(r, (int64_t)k));
                    };
                    sel = below + take(tb, ties);
                    const int64_t ns = max((int64_t)0, min(p1, s_end) - p0);
                    if (ns > 0) sel += (uint32_t)ns - (cnt[2][lane] + take(tb, cnt[3][lane]));
                    const int64_t nr = max((int64_t)0, p1 - max(p0, r_beg));
                    if (nr > 0) sel += (uint32_t)nr - (cnt[4][lane] + take(tb + ties - cnt[5][lane], cnt[5][lane]));
                }
            }
            const uint32_t si = wave_scan_incl(sel);
            if (on) {
                a.rec[(row * nc + c) * 2 + 0] = tb;
                a.rec[(row * nc + c) * 2 + 1] = carry_s + si - sel;
            }
            carry_t += (uint32_t)__builtin_amdgcn_readlane((int)ti, 63);
            carry_s += (uint32_t)__builtin_amdgcn_readlane((int)si, 63);
        }
        if (one) break;
        __syncthreads();   // cnt read before the next block writes it
    }
    if (tid == 0) {
        s_total = carry_s;
        a.count[row] = (int32_t)min((int64_t)carry_s, a.cap);
        a.rowrec[row * 2 + 0] = t;
        a.rowrec[row * 2 + 1] = (int32_t)quota;
    }
    __syncthreads();
    for (int64_t i = (int64_t)s_total + tid; i < a.cap; i += kST) a.idx[row * a.cap + i] = -1;
}

// ---- 3. ordered compaction -------------------------------------------------------
// Exclusive block scan of NV words (each two 16-bit counts); tot = block sums.
template <int NV>
__device__ __forceinline__ void block_scan(uint32_t (&v)[NV], uint32_t (&tot)[NV], uint32_t* sw, int lane, int w) {
    uint32_t inc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) inc[i] = wave_scan_incl(v[i]);
    if (lane == 63)
#pragma unroll
        for (int i = 0; i < NV; ++i) sw[w * NV + i] = inc[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int ww = 0; ww < kWT / 64; ++ww) {
            const uint32_t y = sw[ww * NV + i];
            before += ww < w ? y : 0u;
            all += y;
        }
        v[i] = before + inc[i] - v[i];
        tot[i] = all;
    }
}

__device__ __forceinline__ uint32_t half16(uint32_t v, int j) { return (v >> (16 * (j & 1))) & 0xFFFFu; }

// The lowest r set bits of m.
__device__ __forceinline__ uint32_t lowest_bits(uint32_t m, uint32_t r) {
    uint32_t out = 0;
    for (uint32_t k = 0; k < r && m; ++k) {
        out |= m & (0u - m);
        m &= m - 1u;
    }
    return out;
}

template <int W, int HG, bool VEC>
__global__ __launch_bounds__(kWT, (WideCfg<W, HG>::kCompactWaves)) void k_wide_compact(WideArgs a) {
    using C = WideCfg<W, HG>;
    constexpr int NV = (HG + 1) / 2;
    __shared__ uint32_t sw[2][kWT / 64 * NV];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t c = (int64_t)blockIdx.x % a.nc;
    const WideUnit u = wide_unit<HG>(a, (int)((int64_t)blockIdx.x / a.nc));
    const int64_t n = a.n, nW = n * W;
    const int64_t p0 = c * a.L, p1 = min(n, p0 + a.L);
    const int64_t s_end = min(a.n_sink, n), r_beg = max((int64_t)0, n - a.n_recent);
    int t[HG];
    uint32_t quota[HG], tie_run[HG], sel_run[HG];
    uint32_t q[HG][W];
#pragma unroll
    for (int j = 0; j < HG; ++j) {
        const int64_t row = u.row0 + min(j, u.GH - 1);
        t[j] = a.rowrec[row * 2 + 0];
        quota[j] = (uint32_t)a.rowrec[row * 2 + 1];
        tie_run[j] = a.rec[(row * a.nc + c) * 2 + 0];
        sel_run[j] = a.rec[(row * a.nc + c) * 2 + 1];
#pragma unroll
        for (int k = 0; k < W; ++k) q[j][k] = C::kStore ? 0u : a.q_sigs[row * W + k];
    }
    for (int64_t s0 = p0; s0 < p1; s0 += kTile) {
        const int64_t ps = s0 + kPT * tid;
        const uint32_t nval = (uint32_t)max((int64_t)0, min((int64_t)kPT, p1 - ps));
        const uint32_t valid = (1u << nval) - 1u;
        const uint32_t lo = (uint32_t)max((int64_t)0, min((int64_t)kPT, s_end - ps));
        const uint32_t hi = (uint32_t)max((int64_t)0, min((int64_t)kPT, r_beg - ps));
        const uint32_t win = ((1u << lo) - 1u) | (((1u << kPT) - 1u) & ~((1u << hi) - 1u));
        // per head: positions below t, and ties at t
        uint32_t belm[HG], tiem[HG];
        if constexpr (C::kStore) {
            constexpr int kWords = kPT * HG / 4;   // the positions' bytes, HG per position
            uint32_t db[kWords];
            const uint8_t* src = u.dist + ps * HG;
            if (nval == 0) {
#pragma unroll
                for (int v = 0; v < kWords; ++v) db[v] = 0u;
            } else if constexpr (kWords == 1) {
                db[0] = *reinterpret_cast<const uint32_t*>(src);
            } else if constexpr (kWords == 2) {
                const uint2 y = *reinterpret_cast<const uint2*>(src);
                db[0] = y.x;
                db[1] = y.y;
            } else {
#pragma unroll
                for (int v = 0; v < kWords / 4; ++v) {
                    const u32x4 y = ld16(src + 16 * v);
#pragma unroll
                    for (int e = 0; e < 4; ++e) db[4 * v + e] = y[e];
                }
            }
            bool swar = HG >= 4;
#pragma unroll
            for (int j = 0; j < HG; ++j) swar = swar && t[j] < 255;
            if constexpr (HG >= 4) if (swar) {
                // Four heads at once, per word of a position's bytes: the bytes of heads
                // 4i, 4i+2 (and 4i+1, 4i+3) in the two 16-bit fields of a word, plus
                // 256 - t, carry into bit 8 of the field exactly when the byte >= t
                // (t < 255 here, so every byte is the distance itself); with t + 1, > t.
                // Position k's bit goes to bit 8 + (k mod 8) of the field, one
                // accumulator per half of the tile.
                constexpr int NG = HG >= 4 ? HG / 4 : 1;
                uint32_t ce[NG], ce1[NG], co[NG], co1[NG];
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    auto addend = [&](int ja, int jb, int plus) {
                        const uint32_t ta = (uint32_t)max(0, t[ja] + plus), tb = (uint32_t)max(0, t[jb] + plus);
                        return (256u - ta) | ((256u - tb) << 16);
                    };
                    ce[i] = addend(4 * i, 4 * i + 2, 0);
                    ce1[i] = addend(4 * i, 4 * i + 2, 1);
                    co[i] = addend(4 * i + 1, 4 * i + 3, 0);
                    co1[i] = addend(4 * i + 1, 4 * i + 3, 1);
                }
                uint32_t acc[NG][4][2] = {};   // [group][ge even, gt even, ge odd, gt odd][tile half]
#pragma unroll
                for (int k = 0; k < kPT; ++k) {
#pragma unroll
                    for (int i = 0; i < NG; ++i) {
                        const uint32_t wd = db[k * NG + i];
                        const uint32_t e = wd & 0x00FF00FFu, o = (wd >> 8) & 0x00FF00FFu;
                        const uint32_t r[4] = {e + ce[i], e + ce1[i], o + co[i], o + co1[i]};
#pragma unroll
                        for (int f = 0; f < 4; ++f) acc[i][f][k >> 3] |= (r[f] & 0x01000100u) << (k & 7);
                    }
                }
                // field (0: low, 1: high) of accumulator pair -> 16-bit position mask
                auto mask = [&](const uint32_t (&a2)[2], int field) {
                    const int sh = 8 + 16 * field;
                    return ((a2[0] >> sh) & 0xFFu) | (((a2[1] >> sh) & 0xFFu) << 8);
                };
#pragma unroll
                for (int i = 0; i < NG; ++i) {
#pragma unroll
                    for (int par = 0; par < 2; ++par) {       // even / odd bytes
#pragma unroll
                        for (int field = 0; field < 2; ++field) {
                            const int j = 4 * i + par + 2 * field;
                            const uint32_t ge = mask(acc[i][2 * par], field), gt = mask(acc[i][2 * par + 1], field);
                            belm[j] = ~ge & valid;
                            tiem[j] = ge & ~gt & valid;
                        }
                    }
                }
            }
            if (!swar) {
#pragma unroll
            for (int j = 0; j < HG; ++j) {
                uint32_t bm = 0, tm = 0, cm = 0;
#pragma unroll
                for (int k = 0; k < kPT; ++k) {
                    const int bi = k * HG + j;
                    const int d = (int)((db[bi >> 2] >> (8 * (bi & 3))) & 0xFFu);
                    bm |= (d < t[j] ? 1u : 0u) << k;
                    tm |= (d == t[j] ? 1u : 0u) << k;
                    cm |= (d == 255 ? 1u : 0u) << k;
                }
                cm &= valid;
                if (t[j] >= 255 && cm && j < u.GH) {
                    // a byte of 255 stands for any distance >= 255: resolve it from the codes
                    // (word by word: a rare path, kept out of the registers of the common one)
                    const uint32_t* qj = a.q_sigs + (u.row0 + j) * W;
                    while (cm) {
                        const int k = __builtin_ctz(cm);
                        cm &= cm - 1u;
                        const uint32_t* kp = u.ks + (ps + k) * W;
                        int d = 0;
#pragma unroll 1
                        for (int e = 0; e < W; ++e) d += __builtin_popcount(kp[e] ^ qj[e]);
                        bm = (bm & ~(1u << k)) | ((d < t[j] ? 1u : 0u) << k);
                        tm = (tm & ~(1u << k)) | ((d == t[j] ? 1u : 0u) << k);
                    }
                }
                belm[j] = bm & valid;
                tiem[j] = tm & valid;
            }
            }
        } else {
            uint32_t x[kPT * W];
            if (nval > 0) load_words<kPT * W>(x, u.ks, ps * W, nW, VEC);
#pragma unroll
            for (int j = 0; j < HG; ++j) {
                uint32_t bm = 0, tm = 0;
#pragma unroll
                for (int k = 0; k < kPT; ++k) {
                    const int d = (int)distance<W>(&x[k * W], q[j]);
                    bm |= (d < t[j] ? 1u : 0u) << k;
                    tm |= (d == t[j] ? 1u : 0u) << k;
                }
                belm[j] = bm & valid;
                tiem[j] = tm & valid;
            }
        }
        // tie ranks
        uint32_t v[NV], tot[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            v[i] = (uint32_t)__builtin_popcount(tiem[2 * i]);
            if (2 * i + 1 < HG) v[i] |= (uint32_t)__builtin_popcount(tiem[2 * i + 1]) << 16;
        }
        block_scan<NV>(v, tot, sw[0], lane, w);
        uint32_t selm[HG];
#pragma unroll
        for (int j = 0; j < HG; ++j) {
            const uint32_t before = tie_run[j] + half16(v[j >> 1], j);
            const uint32_t nt = (uint32_t)__builtin_popcount(tiem[j]);
            const uint32_t r = quota[j] > before ? min(quota[j] - before, nt) : 0u;
            const uint32_t top = belm[j] | (r == nt ? tiem[j] : lowest_bits(tiem[j], r));
            selm[j] = (top | win) & valid;
            tie_run[j] += half16(tot[j >> 1], j);
        }
        // output slots
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            v[i] = (uint32_t)__builtin_popcount(selm[2 * i]);
            if (2 * i + 1 < HG) v[i] |= (uint32_t)__builtin_popcount(selm[2 * i + 1]) << 16;
        }
        block_scan<NV>(v, tot, sw[1], lane, w);
#pragma unroll
        for (int j = 0; j < HG; ++j) {
            if (j >= u.GH) continue;
            int64_t slot = (int64_t)sel_run[j] + half16(v[j >> 1], j);
            int32_t* out = a.idx + (u.row0 + j) * a.cap;
            uint32_t m = selm[j];
            while (m) {
                const int k = __builtin_ctz(m);
                m &= m - 1u;
                if (slot < a.cap) out[slot] = (int32_t)(ps + k);
                ++slot;
            }
            sel_run[j] += half16(tot[j >> 1], j);
        }
    }
}

template <int W, int HG, bool VEC>
hipError_t launch_v(const WideArgs& a, hipStream_t st) {
    const int64_t units = (int64_t)a.B * a.Hkv * a.ng;
    const int64_t wgs = units * a.nc;
    if (wgs > 0) hipLaunchKernelGGL((k_wide_hist<W, HG, VEC>), dim3((unsigned)wgs), dim3(kWT), 0, st, a);
    hipLaunchKernelGGL(k_wide_select, dim3((unsigned)((int64_t)a.B * a.Hq)), dim3(kST), 0, st, a);
    if (wgs > 0) hipLaunchKernelGGL((k_wide_compact<W, HG, VEC>), dim3((unsigned)wgs), dim3(kWT), 0, st, a);
    return hipGetLastError();
}
// Codes of W >= 4 words are always aligned vectors (16 W bytes a position).
template <int W, int HG>
hipError_t launch_w(const WideArgs& a, hipStream_t st) {
    if constexpr (W >= 4) return launch_v<W, HG, true>(a, st);
    else return a.vec ? launch_v<W, HG, true>(a, st) : launch_v<W, HG, false>(a, st);
}

template <int W>
hipError_t launch_hg(const WideArgs& a, hipStream_t st) {
    switch (a.HG) {
        case 1: return launch_w<W, 1>(a, st);
        case 2: return launch_w<W, 2>(a, st);
        case 4: return launch_w<W, 4>(a, st);
        case 8: return launch_w<W, 8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

// Workgroups of the histogram and compaction passes one CU holds at once (the smaller).
template <int W, int HG>
int slots_per_cu() {
    int h = 0, c = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&h, k_wide_hist<W, HG, true>, kWT, 0) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, k_wide_compact<W, HG, true>, kWT, 0) != hipSuccess) return 0;
    return min(h, c);
}
template <int W>
int slots_hg(int HG) {
    return HG == 1 ? slots_per_cu<W, 1>() : HG == 2 ? slots_per_cu<W, 2>() : HG == 4 ? slots_per_cu<W, 4>()
                                                                                         : slots_per_cu<W, 8>();
}

}  // namespace

int wide_granule(int W) {
    const int g = W == 1 ? WideCfg<1, 1>::kGranule : W == 2 ? WideCfg<2, 1>::kGranule : WideCfg<4, 1>::kGranule;
    return max(g, kTile);   // both divide kWideMaxL; a chunk is whole loop turns and whole tiles
}

int wide_slots_per_cu(int W, int HG) {
    switch (W) {
        case 1: return slots_hg<1>(HG);
        case 2: return slots_hg<2>(HG);
        case 4: return slots_hg<4>(HG);
        case 8: return slots_hg<8>(HG);
        case 16: return slots_hg<16>(HG);
        default: return 0;
    }
}

int wide_group(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }

hipError_t launch_topk_wide(const WideArgs& a, hipStream_t st) {
    if (a.B <= 0) return hipSuccess;
    if (a.HG != wide_group(a.G) || a.ng != (a.G + a.HG - 1) / a.HG || a.L < 16 || a.L > kWideMaxL ||
        a.L % 16 != 0 || a.nc != (a.n + a.L - 1) / a.L || a.dstride < ((a.n + 15) / 16 * 16) * a.HG ||
        a.dstride % 16 != 0)
        return hipErrorInvalidValue;
    if ((int64_t)a.B * a.Hkv * a.ng * a.nc > INT32_MAX || (int64_t)a.B * a.Hq > INT32_MAX) return hipErrorInvalidValue;
    switch (a.W) {
        case 1: return launch_hg<1>(a, st);
        case 2: return launch_hg<2>(a, st);
        case 4: return launch_hg<4>(a, st);
        case 8: return launch_hg<8>(a, st);
        case 16: return launch_hg<16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lcda
