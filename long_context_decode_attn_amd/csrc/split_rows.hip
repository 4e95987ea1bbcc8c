// split_rows.hip - split-KV partials when many query rows read one KV head: a
// shared document whose K/V every batch item's G query heads attend to
// ("Nectar: Neural Estimation of Cached-Token Attention via Regression", slide
// "A fixed document is expensive to read repeatedly": the document's K/V are
// fixed and read for every new query).
//
// A workgroup owns 64 query rows (4 wavefronts x 16) of one KV head and one
// token range.  Each 32-token block of that range is brought into an LDS ring
// once (buffer loads straight to LDS, no registers held while in flight), then
// every wavefront reads the whole block back in the MFMA lane layout and runs
// the 16-row tile on its own rows: HBM reads each block once for all 64 rows,
// and each wavefront keeps only one 16-row tile of state.
//
// Ring: kSlots slots of one block; the block kSlots - 1 ahead is requested
// while the current one is computed.  Each wavefront requests 4 of the block's
// 16 pieces (lane l of piece i lands at slot + 1024*i + 16*l, the place every
// wavefront's lane l later reads it from).  The loop's barrier is a bare
// s_barrier: completion of the ring's own requests is tracked with explicit
// vmcnt waits, and every other memory operation of the loop is an LDS read
// that waits for itself.  A block is ready when every
// wavefront's own pieces have landed (vmcnt) and all have passed the barrier;
// a slot is refilled only after that barrier, when every wavefront has
// finished reading the block it held.  Requests past the end of the range use
// an empty buffer resource, so every step has the same requests outstanding
// and none of them reads memory.

#include "common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace lcda {
namespace {

constexpr int kSlotBytes = 16384;
constexpr int kPieces = 4;           // pieces (of 16) each wavefront requests per block
constexpr int kRowsPerGroup = 16 * kWaves;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt vmcnt(kPieces * (ahead - 1)): this wavefront's pieces of the
// current block have landed; those of the ahead - 1 younger blocks may still
// be in flight.  (gfx9 encoding; expcnt and lgkmcnt at their maxima.)
template <int AHEAD>
constexpr int vmcnt_ring() {
    static_assert(kPieces * (AHEAD - 1) < 16, "vmcnt low field");
    return 0x0F70 | (kPieces * (AHEAD - 1));
}

// Query fragments of a wavefront's 16*NT rows (row c16 of each tile) and a fresh state.
template <int NT>
__device__ __forceinline__ void load_rows_q(WaveState<NT>& st, const SplitArgs& a, int rows_w, int bkv, int h, int j,
                                            int c16) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        const int r = rows_w + 16 * rt + c16;
        if (r < a.rows) {
            const int b = a.shared ? r / a.G : bkv;
            const int g = a.shared ? r % a.G : r;
            const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + h * a.G + g) * kD + 8 * j;
#pragma unroll
            for (int c = 0; c < 4; ++c) st.q[rt][c] = as_bf16x8(ld16(qp + 32 * c));
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) st.q[rt][c] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) st.o[rt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m[rt] = kNoMax;
        st.l[rt] = 0.f;
    }
}

// A wavefront's 16*NT rows out: per tile, m per row c16 (shared by the lane
// groups), l summed over them; o[rt][nb][i] is row 16*rt + 4j + i, column
// 8*c16 + nb.  Direct: finished rows (with the optional virtual pair); else the
// (row, split) partial state.
template <int NT>
__device__ __forceinline__ void write_rows(const WaveState<NT>& st, const SplitArgs& a, int rows_w, int bkv, int h,
                                           int split, int j, int c16, int lane, bool direct) {
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        float l = st.l[rt];
        l = sum_xor32(sum_xor16(l));
        const float m = st.m[rt];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 4 * j + i;
            const int r = rows_w + 16 * rt + rr;
            const float M = __shfl(m, rr, 64);   // row rr's state lives in lane rr (j = 0)
            const float L = __shfl(l, rr, 64);
            if (r >= a.rows) continue;
            const int b = a.shared ? r / a.G : bkv;
            const int g = a.shared ? r % a.G : r;
            const int64_t bhq = (int64_t)b * a.Hq + h * a.G + g;
            if (direct) {
                const bool virt = a.alpha_in != nullptr && a.alpha_in[bhq] > -INFINITY;
                const float al = virt ? a.alpha_in[bhq] : -INFINITY;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    const int c = 8 * c16 + nb;
                    finish_row(a, bhq, c, M, L, st.o[rt][nb][i], virt, al, virt ? a.a_in[bhq * kD + c] : 0.f);
                }
            } else {
                const int64_t slot = bhq * a.splits + split;
                float* dst = a.acc + slot * kD + 8 * c16;
                *reinterpret_cast<f32x4*>(dst) =
                    f32x4{st.o[rt][0][i], st.o[rt][1][i], st.o[rt][2][i], st.o[rt][3][i]};
                *reinterpret_cast<f32x4*>(dst + 4) =
                    f32x4{st.o[rt][4][i], st.o[rt][5][i], st.o[rt][6][i], st.o[rt][7][i]};
                if (c16 == 0) a.ml[slot] = make_float2(M, L);
            }
        }
    }
}

// This wavefront's pieces of block t (rows [t, t + 32) of the head) into `slot`.
template <bool NTL>
__device__ __forceinline__ void request_block(char* slot, const uint16_t* kh, const uint16_t* vh, int64_t t,
                                              int64_t n_eff, bool live, int w, uint32_t koff, uint32_t voff) {
    const int64_t left = n_eff - t;
    const int nrec = live ? (int)(left < kBlock ? left : kBlock) * kD * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kh + t * kD), 0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vh + t * kD), 0, nrec, kRsrcWord3);
    constexpr int aux = NTL ? 2 : 0;   // nontemporal
    // Wavefront w requests pieces w + 4p: K (half p, d chunk w) for p = 0, 1 and
    // V (row set e = w + 4(p - 2)) for p = 2, 3, the same code in every wavefront.
    const uint32_t kw = koff + 64u * w, vw = voff + 256u * w;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(slot + 1024 * w), 16, kw, 0, 0, aux);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(slot + 1024 * (w + 4)), 16, kw + 4096, 0, 0, aux);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(slot + 1024 * (w + 8)), 16, vw, 0, 0, aux);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(slot + 1024 * (w + 12)), 16, vw + 4096, 0, 0, aux);
}

// This lane's 16 pieces of a slot (addr = slot + 16*lane) into registers; the
// asm waits for its own LDS reads.  The outputs are early-clobber: a read's
// destination must never be the address register a later read of the block
// still uses (the reads complete asynchronously).
__device__ __forceinline__ void read_block(BlockRegs& r, uint32_t addr) {
    asm volatile(
        "ds_read_b128 %0, %16 offset:0\n\t"
        "ds_read_b128 %1, %16 offset:1024\n\t"
        "ds_read_b128 %2, %16 offset:2048\n\t"
        "ds_read_b128 %3, %16 offset:3072\n\t"
        "ds_read_b128 %4, %16 offset:4096\n\t"
        "ds_read_b128 %5, %16 offset:5120\n\t"
        "ds_read_b128 %6, %16 offset:6144\n\t"
        "ds_read_b128 %7, %16 offset:7168\n\t"
        "ds_read_b128 %8, %16 offset:8192\n\t"
        "ds_read_b128 %9, %16 offset:9216\n\t"
        "ds_read_b128 %10, %16 offset:10240\n\t"
        "ds_read_b128 %11, %16 offset:11264\n\t"
        "ds_read_b128 %12, %16 offset:12288\n\t"
        "ds_read_b128 %13, %16 offset:13312\n\t"
        "ds_read_b128 %14, %16 offset:14336\n\t"
        "ds_read_b128 %15, %16 offset:15360\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.k[0][0]), "=&v"(r.k[0][1]), "=&v"(r.k[0][2]), "=&v"(r.k[0][3]), "=&v"(r.k[1][0]),
          "=&v"(r.k[1][1]), "=&v"(r.k[1][2]), "=&v"(r.k[1][3]), "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.v[2]),
          "=&v"(r.v[3]), "=&v"(r.v[4]), "=&v"(r.v[5]), "=&v"(r.v[6]), "=&v"(r.v[7])
        : "v"(addr)
        : "memory");
}

// Block t of a head's rows straight into registers (buffer loads; rows at or
// past n_eff read as zero, and live = false issues an empty request).
// Returns the rows of the block that exist.
template <bool NTL>
__device__ __forceinline__ int load_rows_block(BlockRegs& r, const uint16_t* kh, const uint16_t* vh, int64_t t,
                                               int64_t n_eff, bool live, uint32_t koff, uint32_t voff) {
    const int64_t left = n_eff - t;
    const int valid = (int)(left < kBlock ? left : kBlock);
    const int nrec = live ? valid * kD * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kh + t * kD), 0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vh + t * kD), 0, nrec, kRsrcWord3);
    constexpr int aux = NTL ? 2 : 0;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            r.k[tb][c] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 4096 * tb + 64 * c, 0, aux);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        r.v[e] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + (e < 4 ? 0 : 4096) + 256 * (e & 3), 0, aux);
    return valid;
}

// Local tokens in the same pass (the fused decode step over a shared document):
// each batch item's private tokens are an extra range attended to by its own G
// rows only.  A wavefront's 16 rows belong to items i0 .. i1; the local blocks
// of those items, numbered k = (item - i0) * nbl + block, go to the splits in
// turn (split s takes k = s, s + splits, ...), so each wavefront runs about
// one extra block, with the rows of other items masked.
struct LocalWork {
    int i0 = 0, nbl = 1;
    int64_t count = 0;   // local blocks of this wavefront's items
};

__device__ __forceinline__ LocalWork local_work(const SplitArgs& a, int rows_w) {
    LocalWork lw;
    if (a.k2 == nullptr || a.n2 <= 0 || rows_w >= a.rows) return lw;
    lw.i0 = rows_w / a.G;
    const int i1 = (min(rows_w + 16, a.rows) - 1) / a.G;
    lw.nbl = (int)((a.n2 + kBlock - 1) / kBlock);
    lw.count = (int64_t)(i1 - lw.i0 + 1) * lw.nbl;
    return lw;
}

template <bool NTL>
__device__ __forceinline__ int load_local_block(BlockRegs& r, const SplitArgs& a, int h, const LocalWork& lw, int64_t k,
                                                uint32_t koff, uint32_t voff) {
    const int item = lw.i0 + (int)(k / lw.nbl);
    const int64_t t = (int64_t)kBlock * (k % lw.nbl);
    const int64_t n_item = a.n2_b ? min(max((int64_t)a.n2_b[item], (int64_t)0), a.n2) : a.n2;
    const int64_t off = (int64_t)item * a.kv2_batch_stride + (int64_t)h * a.n2 * kD;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k2) + off;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v2) + off;
    const bool live = t < n_item;
    return load_rows_block<NTL>(r, kh, vh, live ? t : 0, n_item, live, koff, voff) * (live ? 1 : 0);
}

// SLOTS: ring slots (SLOTS - 1 blocks ahead).  WPE: waves per SIMD the
// register allocation leaves room for.  DIRECT: one split per unit, rows
// finished in place.  LOCAL: the rows' local tokens (a.k2, a.v2) are attended
// to in the same pass.
template <int SLOTS, bool NTL, int WPE, bool DIRECT, bool LOCAL = false>
__global__ __launch_bounds__(64 * kWaves, WPE) void k_split_rows(SplitArgs a) {
    constexpr int kSlots = SLOTS, kAhead = SLOTS - 1;
    __shared__ __attribute__((aligned(16))) char ring[kSlots][kSlotBytes];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane >> 4, c16 = lane & 15;
    const uint32_t koff = 256u * c16 + 16u * j;
    const uint32_t voff = 1024u * j + 16u * c16;
    const int split = blockIdx.x, h = blockIdx.y;
    const int bkv = blockIdx.z / a.row_groups, rg = blockIdx.z % a.row_groups;
    const int rows_w = rg * kRowsPerGroup + 16 * w;   // this wavefront's first row

    const int64_t n_eff = a.n_b ? min((int64_t)a.n_b[bkv], a.n) : a.n;
    const int64_t head_off = (int64_t)bkv * a.kv_batch_stride + (int64_t)h * a.n * kD;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k) + head_off;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v) + head_off;
    const int64_t t_begin = (int64_t)split * a.blocks_per_split * kBlock;
    const int64_t t_end = min(n_eff, t_begin + (int64_t)a.blocks_per_split * kBlock);
    const int nblk = t_end > t_begin ? (int)((t_end - t_begin + kBlock - 1) / kBlock) : 0;

    // The first local block is requested with the query fragments; it lands
    // while the document's blocks stream.
    LocalWork lw;
    BlockRegs lr;
    int lvalid = 0;
    if (LOCAL) {
        lw = local_work(a, rows_w);
        if (split < lw.count) lvalid = load_local_block<NTL>(lr, a, h, lw, split, koff, voff);
    }
    WaveState<1> st;
    load_rows_q(st, a, rows_w, bkv, h, j, c16);
    wait_vm_all();   // only the ring's requests are outstanding from here on

    const uint32_t lane_off = lds_addr(ring[0]) + 16 * lane;
    if (nblk > 0) {
#pragma unroll
        for (int k = 0; k < kAhead; ++k) {
            const int kk = min(k, nblk - 1);
            request_block<NTL>(ring[k], kh, vh, t_begin + (int64_t)kBlock * kk, n_eff, k < nblk, w, koff, voff);
        }
        for (int k = 0; k < nblk; ++k) {
            __builtin_amdgcn_s_waitcnt(vmcnt_ring<kAhead>());   // this wavefront's pieces of block k
            // Everyone's pieces of block k have landed, and every wavefront has read block k - 1.  A bare
            // barrier: a fenced one would also wait for the blocks still in flight.
            __builtin_amdgcn_s_barrier();
            const int kn = k + kAhead;
            request_block<NTL>(ring[kn % kSlots], kh, vh, t_begin + (int64_t)kBlock * min(kn, nblk - 1), n_eff,
                               kn < nblk, w, koff, voff);
            BlockRegs r;
            read_block(r, lane_off + (k % kSlots) * kSlotBytes);
            const int64_t t = t_begin + (int64_t)kBlock * k;
            const int64_t left = n_eff - t;
            compute_block<1>(st, r, (int)(left < kBlock ? left : kBlock), a.scale_log2, j, c16);
        }
    }
    wait_vm_all();   // the empty requests past the end

    if (LOCAL) {
        const int r = rows_w + c16;
        for (int64_t k = split; k < lw.count; k += a.splits) {
            if (k != split) {
                lvalid = load_local_block<NTL>(lr, a, h, lw, k, koff, voff);
                wait_vm_all();
            }
            const int item = lw.i0 + (int)(k / lw.nbl);
            if (lvalid > 0) compute_block<1>(st, lr, lvalid, a.scale_log2, j, c16, r < a.rows && r / a.G == item);
        }
    }

    write_rows(st, a, rows_w, bkv, h, split, j, c16, lane, DIRECT);

    // Several splits: the combine pass merges them (a unit here has 64 rows x
    // splits partial states, too many for the one workgroup that would finish
    // last to gather quickly).
}

// ---- pair variant -------------------------------------------------------------
// The 64 rows as two halves of 32 (two 16-row tiles per wavefront); the two
// wavefronts of a half take alternate blocks (wavefront w: half w & 1, block
// parity w >> 1), so every block is read back from LDS by two wavefronts
// instead of four, and each wavefront's block chain carries two independent
// tiles.  The ring advances by a pair of blocks per barrier: pair k (blocks 2k,
// 2k + 1) is computed while blocks 2k + 2 .. 2k + 4 are in flight, in a ring
// of five slots (block b in slot b % 5).  At the end the two wavefronts of a
// half merge their states through LDS (exactly, by their maxima) and one of
// them writes the half's rows.
constexpr int kPairSlots = 5;
constexpr int kPairRows = 32;

// s_waitcnt vmcnt(kPieces): the pair's blocks have landed; the one younger
// block may still be in flight.
constexpr int vmcnt_pair() { return 0x0F70 | kPieces; }

// Local blocks of a wavefront's 32 rows: as local_work, for the items of rows
// rows_w .. rows_w + 31.
__device__ __forceinline__ LocalWork local_work_rows(const SplitArgs& a, int rows_w, int nrows) {
    LocalWork lw;
    if (a.k2 == nullptr || a.n2 <= 0 || rows_w >= a.rows) return lw;
    lw.i0 = rows_w / a.G;
    const int i1 = (min(rows_w + nrows, a.rows) - 1) / a.G;
    lw.nbl = (int)((a.n2 + kBlock - 1) / kBlock);
    lw.count = (int64_t)(i1 - lw.i0 + 1) * lw.nbl;
    return lw;
}

// One 16-row tile of a two-tile state through the one-tile block computation
// (a local block that only one item's rows see, so at most the tiles holding
// them run).
template <int RT>
__device__ __forceinline__ void compute_tile(WaveState<2>& st, const BlockRegs& r, int valid, float scale, int j,
                                             int c16, bool ok) {
    WaveState<1> t;
#pragma unroll
    for (int c = 0; c < 4; ++c) t.q[0][c] = st.q[RT][c];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) t.o[0][nb] = st.o[RT][nb];
    t.m[0] = st.m[RT];
    t.l[0] = st.l[RT];
    compute_block<1>(t, r, valid, scale, j, c16, ok ? 1 : 0);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) st.o[RT][nb] = t.o[0][nb];
    st.m[RT] = t.m[0];
    st.l[RT] = t.l[0];
}

template <bool NTL, bool DIRECT, bool LOCAL>
__global__ __launch_bounds__(64 * kWaves, 2) void k_split_rows_pair(SplitArgs a) {
    static_assert(kWaves == 4 && 2 * kPairRows == kRowsPerGroup, "two halves of two wavefronts");
    __shared__ __attribute__((aligned(16))) char ring[kPairSlots][kSlotBytes];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = w & 1, par = w >> 1;
    const int j = lane >> 4, c16 = lane & 15;
    const uint32_t koff = 256u * c16 + 16u * j;
    const uint32_t voff = 1024u * j + 16u * c16;
    const int split = blockIdx.x, h = blockIdx.y;
    const int bkv = blockIdx.z / a.row_groups, rg = blockIdx.z % a.row_groups;
    const int rows_w = rg * kRowsPerGroup + kPairRows * half;   // this wavefront's first row

    const int64_t n_eff = a.n_b ? min((int64_t)a.n_b[bkv], a.n) : a.n;
    const int64_t head_off = (int64_t)bkv * a.kv_batch_stride + (int64_t)h * a.n * kD;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k) + head_off;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v) + head_off;
    const int64_t t_begin = (int64_t)split * a.blocks_per_split * kBlock;
    const int64_t t_end = min(n_eff, t_begin + (int64_t)a.blocks_per_split * kBlock);
    const int nblk = t_end > t_begin ? (int)((t_end - t_begin + kBlock - 1) / kBlock) : 0;

    // Local blocks of the half's items go to the 2 * splits wavefronts of the
    // half in turn: wavefront (split, par) takes k = 2*split + par, then every
    // 2 * splits-th.  The first two are requested with the query fragments and
    // computed while the ring's first blocks are in flight (the registers of
    // two blocks fit before the document loop, not across it); any further
    // ones run after the loop.
    LocalWork lw;
    BlockRegs lr, lr2;
    int lvalid = 0, lvalid2 = 0;
    const int64_t lfirst = 2 * (int64_t)split + par, lstep = 2 * (int64_t)a.splits;
    if (LOCAL) {
        lw = local_work_rows(a, rows_w, kPairRows);
        if (lfirst < lw.count) lvalid = load_local_block<NTL>(lr, a, h, lw, lfirst, koff, voff);
        if (lfirst + lstep < lw.count) lvalid2 = load_local_block<NTL>(lr2, a, h, lw, lfirst + lstep, koff, voff);
    }
    WaveState<2> st;
    load_rows_q(st, a, rows_w, bkv, h, j, c16);
    wait_vm_all();   // only the ring's requests are outstanding from here on

    // A local block k (in registers r, valid rows v): only the tiles holding
    // the item's rows run (the item's rows are consecutive, so this is
    // uniform), with the other rows masked.
    auto local_block = [&](int64_t k, const BlockRegs& r, int v) {
        if (v <= 0) return;
        const int item = lw.i0 + (int)(k / lw.nbl);
        const int r0 = rows_w + c16, r1 = rows_w + 16 + c16;
        const int first = item * a.G - rows_w, last = first + a.G - 1;
        if (first < 16) compute_tile<0>(st, r, v, a.scale_log2, j, c16, r0 < a.rows && r0 / a.G == item);
        if (last >= 16) compute_tile<1>(st, r, v, a.scale_log2, j, c16, r1 < a.rows && r1 / a.G == item);
    };

    const uint32_t lane_off = lds_addr(ring[0]) + 16 * lane;
    if (nblk > 0) {
#pragma unroll
        for (int k = 0; k < kPairSlots - 2; ++k) {
            const int kk = min(k, nblk - 1);
            request_block<NTL>(ring[k], kh, vh, t_begin + (int64_t)kBlock * kk, n_eff, k < nblk, w, koff, voff);
        }
    }
    if (LOCAL && lfirst < lw.count) local_block(lfirst, lr, lvalid);
    if (LOCAL && lfirst + lstep < lw.count) local_block(lfirst + lstep, lr2, lvalid2);
    if (nblk > 0) {
        const int npairs = (nblk + 1) / 2;
        for (int k = 0; k < npairs; ++k) {
            __builtin_amdgcn_s_waitcnt(vmcnt_pair());   // this wavefront's pieces of blocks 2k, 2k + 1
            // Everyone's pieces of the pair have landed, and every wavefront has read pair k - 1.
            __builtin_amdgcn_s_barrier();
#pragma unroll
            for (int u = 0; u < 2; ++u) {   // into the slots of pair k - 1
                const int kn = 2 * k + kPairSlots - 2 + u;
                request_block<NTL>(ring[kn % kPairSlots], kh, vh, t_begin + (int64_t)kBlock * min(kn, nblk - 1),
                                   n_eff, kn < nblk, w, koff, voff);
            }
            const int kb = 2 * k + par;
            if (kb < nblk) {
                BlockRegs r;
                read_block(r, lane_off + (kb % kPairSlots) * kSlotBytes);
                const int64_t left = n_eff - (t_begin + (int64_t)kBlock * kb);
                compute_block<2>(st, r, (int)(left < kBlock ? left : kBlock), a.scale_log2, j, c16);
            }
        }
    }
    wait_vm_all();   // the empty requests past the end

    if (LOCAL) {
        for (int64_t k = lfirst + 2 * lstep; k < lw.count; k += lstep) {
            lvalid = load_local_block<NTL>(lr, a, h, lw, k, koff, voff);
            wait_vm_all();
            local_block(k, lr, lvalid);
        }
    }

    // Merge the two block parities of each half: parity 1 leaves its state in
    // the ring (no longer in use), parity 0 folds it into its own.
    __builtin_amdgcn_s_barrier();   // every wavefront is done reading the ring
    float* xo = reinterpret_cast<float*>(&ring[0][0]) + half * (2 * 8 * 4 * 64);   // [rt][nb][i][lane]
    float2* xml = reinterpret_cast<float2*>(&ring[2][0]) + half * (2 * 64);          // [rt][lane]
    if (par == 1) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
            for (int nb = 0; nb < 8; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) xo[((rt * 8 + nb) * 4 + i) * 64 + lane] = st.o[rt][nb][i];
            xml[rt * 64 + lane] = make_float2(st.m[rt], st.l[rt]);
        }
    }
    __syncthreads();
    if (par == 0) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float2 o1 = xml[rt * 64 + lane];   // row c16's max and this lane's sum, parity 1
            const float M = fmaxf(st.m[rt], o1.x);
            const float w0 = fast_exp2(st.m[rt] - M), w1 = fast_exp2(o1.x - M);
            st.m[rt] = M;
            st.l[rt] = st.l[rt] * w0 + o1.y * w1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a0 = __shfl(w0, 4 * j + i, 64), a1 = __shfl(w1, 4 * j + i, 64);   // row 4j + i
#pragma unroll
                for (int nb = 0; nb < 8; ++nb)
                    st.o[rt][nb][i] = st.o[rt][nb][i] * a0 + xo[((rt * 8 + nb) * 4 + i) * 64 + lane] * a1;
            }
        }
        write_rows(st, a, rows_w, bkv, h, split, j, c16, lane, DIRECT);
    }
}

// ---- register variant ---------------------------------------------------------
// The same split of rows over wavefronts, without LDS: every wavefront requests
// the whole block into its own registers (buffer loads, one block ahead); the
// four requests of a block go to the same addresses at about the same time and
// are served once from the caches (cached loads), so HBM still reads each
// block once.
template <bool NTL, int WPE, bool DIRECT>
__global__ __launch_bounds__(64 * kWaves, WPE) void k_split_rows_regs(SplitArgs a) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane >> 4, c16 = lane & 15;
    const uint32_t koff = 256u * c16 + 16u * j;
    const uint32_t voff = 1024u * j + 16u * c16;
    const int split = blockIdx.x, h = blockIdx.y;
    const int bkv = blockIdx.z / a.row_groups, rg = blockIdx.z % a.row_groups;
    const int rows_w = rg * kRowsPerGroup + 16 * w;

    const int64_t n_eff = a.n_b ? min((int64_t)a.n_b[bkv], a.n) : a.n;
    const int64_t head_off = (int64_t)bkv * a.kv_batch_stride + (int64_t)h * a.n * kD;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k) + head_off;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v) + head_off;
    const int64_t t_begin = (int64_t)split * a.blocks_per_split * kBlock;
    const int64_t t_end = min(n_eff, t_begin + (int64_t)a.blocks_per_split * kBlock);
    const int nblk = t_end > t_begin ? (int)((t_end - t_begin + kBlock - 1) / kBlock) : 0;

    WaveState<1> st;
    load_rows_q(st, a, rows_w, bkv, h, j, c16);
    BlockRegs buf[2];
    int valid[2] = {0, 0};
    if (nblk > 0) valid[0] = load_rows_block<NTL>(buf[0], kh, vh, t_begin, n_eff, true, koff, voff);
    wait_vm_all();   // the query fragments and the first block

    for (int k = 0; k < nblk;) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (k < nblk) {
                const int kn = k + 1;
                valid[u ^ 1] = load_rows_block<NTL>(buf[u ^ 1], kh, vh, t_begin + (int64_t)kBlock * min(kn, nblk - 1),
                                                    n_eff, kn < nblk, koff, voff);
                __builtin_amdgcn_sched_barrier(0);
                compute_block<1>(st, buf[u], valid[u], a.scale_log2, j, c16);
                ++k;
            }
        }
    }
    wait_vm_all();
    write_rows(st, a, rows_w, bkv, h, split, j, c16, lane, DIRECT);
}

}  // namespace

int split_rows_per_group() { return kRowsPerGroup; }

hipError_t launch_split_rows(const SplitPlan& p, const SplitArgs& a, hipStream_t st) {
    dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(64 * kWaves);
    const int variant = (int)tuning().rows_variant;
    if (variant == 8) {   // two-tile wavefronts on alternate blocks
        if (a.k2 != nullptr && a.direct) hipLaunchKernelGGL((k_split_rows_pair<true, true, true>), grid, block, 0, st, a);
        else if (a.k2 != nullptr) hipLaunchKernelGGL((k_split_rows_pair<true, false, true>), grid, block, 0, st, a);
        else if (a.direct) hipLaunchKernelGGL((k_split_rows_pair<true, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_split_rows_pair<true, false, false>), grid, block, 0, st, a);
        return hipGetLastError();
    }
    if (a.k2 != nullptr) {   // local tokens in the same pass: the default ring variant (or the 5-slot one)
        if (a.direct) hipLaunchKernelGGL((k_split_rows<4, true, 1, true, true>), grid, block, 0, st, a);
        else if (variant == 7) hipLaunchKernelGGL((k_split_rows<5, true, 2, false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_split_rows<4, true, 2, false, true>), grid, block, 0, st, a);
        return hipGetLastError();
    }
    if (a.direct) hipLaunchKernelGGL((k_split_rows<4, true, 1, true>), grid, block, 0, st, a);
    else if (variant == 1) hipLaunchKernelGGL((k_split_rows<3, true, 3, false>), grid, block, 0, st, a);
    else if (variant == 2) hipLaunchKernelGGL((k_split_rows<3, true, 2, false>), grid, block, 0, st, a);
    else if (variant == 3) hipLaunchKernelGGL((k_split_rows<2, true, 3, false>), grid, block, 0, st, a);
    else if (variant == 4) hipLaunchKernelGGL((k_split_rows_regs<false, 2, false>), grid, block, 0, st, a);
    else if (variant == 5) hipLaunchKernelGGL((k_split_rows_regs<true, 2, false>), grid, block, 0, st, a);
    else if (variant == 6) hipLaunchKernelGGL((k_split_rows_regs<false, 1, false>), grid, block, 0, st, a);
    else if (variant == 7) hipLaunchKernelGGL((k_split_rows<5, true, 2, false>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_split_rows<4, true, 2, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace lcda
