// split_mfma.hip - split-KV decode attention partials for bf16 K/V on CDNA4
// matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Computes, for every query row of a work unit and every token range (split),
// the partial softmax state m, l, acc of "Nectar: Neural Estimation of
// Cached-Token Attention via Regression", Eq. (3.1), in base-2 units:
//   x_j = (q . k_j) * log2(e) / sqrt(d),  m = max_j x_j,
//   l = sum_j 2^(x_j - m),  acc = sum_j 2^(x_j - m) v_j.
// Ranges are merged exactly afterwards through their log-normalizers.
//
// Mapping onto the hardware
// - A wavefront owns 16*NT query rows (the GQA group, or every (batch, group)
//   pair reading one shared document) and walks 32-token blocks.
// - S^T = K Q^T: K rows are the MFMA A operand (16 tokens x 32 d per
//   instruction), loaded straight from HBM with 16-byte loads; Q^T (the B
//   operand) stays in registers for the whole wave.
// - O += P V: P is already in A-operand layout in the lane that computed it (the
//   token order inside the 32-token block is permuted to make that so, and V is
//   read in the same order), split into bf16 hi + lo halves so the product keeps
//   ~16 significant bits of P.  The V operand needs 8 tokens of one d column
//   per lane: each lane loads 8 full-row 16-byte pieces (4 rows per load
//   instruction, 256 contiguous bytes per row) and transposes them in registers
//   with v_perm_b32; the d columns of the output are permuted accordingly
//   (column n of block nb is d = 8n + nb).
// - Online softmax with a lazy rescale: the running max only moves when a row's
//   block max exceeds it by more than 2^8, which keeps every weight <= 256.
// - The next block's loads are issued before the current block is computed.
// - The 4 waves of a workgroup interleave blocks of the split and merge their
//   states through LDS, so each (row, split) slot is written once.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

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

// Token t of the row's token range lives in segment 1 (kh, vh) when t < n_c,
// else at t - n_c in segment 2 (kh2, vh2).  A block entirely on one side uses
// that side's base; only a block that straddles n_c selects per lane.
struct Segs {
    const uint16_t* kh;
    const uint16_t* vh;
    const uint16_t* kh2;
    const uint16_t* vh2;
    int64_t n_c;
};

template <bool NTL, bool FUSED>
__device__ __forceinline__ const uint16_t* row_ptr(const Segs& sg, bool second, int64_t tok, bool k) {
    if (!FUSED) return (k ? sg.kh : sg.vh) + tok * kD;
    return second ? (k ? sg.kh2 : sg.vh2) + (tok - sg.n_c) * kD : (k ? sg.kh : sg.vh) + tok * kD;
}

template <bool NTL, bool FUSED>
__device__ __forceinline__ void load_block(BlockRegs& r, const Segs& sg, int64_t t, int64_t last, int j, int c16) {
    // uniform per block: 0 = all in segment 1, 1 = all in segment 2, 2 = straddles
    const int side = !FUSED ? 0 : (t + kBlock <= sg.n_c ? 0 : (t >= sg.n_c ? 1 : 2));
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int64_t tok = min(t + 16 * tb + c16, last);
        const bool second = side == 1 || (side == 2 && tok >= sg.n_c);
        const uint16_t* p = row_ptr<NTL, FUSED>(sg, second, tok, true) + 8 * j;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.k[tb][c] = ld16s<NTL>(p + 32 * c);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t tok = min(t + tok_of(j, e), last);
        const bool second = side == 1 || (side == 2 && tok >= sg.n_c);
        r.v[e] = ld16s<NTL>(row_ptr<NTL, FUSED>(sg, second, tok, false) + 8 * c16);
    }
}

// ---- LDS-ring variant -------------------------------------------------------
// Each wave owns two 16 KB LDS slots.  A block is requested straight into a
// slot with global->LDS loads (no VGPRs are held while it is in flight): lane l
// of load instruction i writes its 16 bytes at slot + 1024*i + 16*l, and later
// reads them back from the same place, so the register layout after the read
// is exactly the one load_block produces.  The wait for a slot's data is an
// explicit vmcnt, and the read of the slot is a single asm block that waits for
// its own LDS reads, so the compiler never has to guess which slot a wait is
// for.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kSlotBytes = 16384;
constexpr int kVmcnt16 = 0x4F70;   // s_waitcnt vmcnt(16) (gfx9 encoding; other counters at maxima)

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <bool NTL, bool FUSED>
__device__ __forceinline__ void dma_block(char* slot, const Segs& sg, int64_t t, int64_t last, int j, int c16) {
    const int side = !FUSED ? 0 : (t + kBlock <= sg.n_c ? 0 : (t >= sg.n_c ? 1 : 2));
    constexpr int aux = NTL ? 2 : 0;   // nontemporal
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int64_t tok = min(t + 16 * tb + c16, last);
        const bool second = side == 1 || (side == 2 && tok >= sg.n_c);
        const uint16_t* p = row_ptr<NTL, FUSED>(sg, second, tok, true) + 8 * j;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            __builtin_amdgcn_global_load_lds((const void*)(p + 32 * c), (lds_ptr_t)(slot + 1024 * (4 * tb + c)), 16, 0,
                                             aux);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t tok = min(t + tok_of(j, e), last);
        const bool second = side == 1 || (side == 2 && tok >= sg.n_c);
        __builtin_amdgcn_global_load_lds((const void*)(row_ptr<NTL, FUSED>(sg, second, tok, false) + 8 * c16),
                                         (lds_ptr_t)(slot + 1024 * (8 + e)), 16, 0, aux);
    }
}

// This lane's 16 pieces of a slot (addr = slot + 16*lane) into registers.
__device__ __forceinline__ void lds_read_block(BlockRegs& r, uint32_t addr) {
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
        : "=v"(r.k[0][0]), "=v"(r.k[0][1]), "=v"(r.k[0][2]), "=v"(r.k[0][3]), "=v"(r.k[1][0]), "=v"(r.k[1][1]),
          "=v"(r.k[1][2]), "=v"(r.k[1][3]), "=v"(r.v[0]), "=v"(r.v[1]), "=v"(r.v[2]), "=v"(r.v[3]), "=v"(r.v[4]),
          "=v"(r.v[5]), "=v"(r.v[6]), "=v"(r.v[7])
        : "v"(addr)
        : "memory");
}

template <int NT>
struct WaveState {
    bf16x8 q[NT][4];
    f32x4 o[NT][8];
    float m[NT];
    float l[NT];
};

template <int NT>
__device__ __forceinline__ void compute_block(WaveState<NT>& st, const BlockRegs& r, int64_t t,
                                              int64_t n_eff, float scale, int j, int c16) {
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
    // Scores: s[rt][tb][i] is token t + 16*tb + 4*j + i of row 16*rt + c16.
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
    const bool full = (t + kBlock <= n_eff);
    float bm[NT];
    bool need = false;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[rt][tb][i] * scale;
                if (!full && t + 16 * tb + 4 * j + i >= n_eff) x = -INFINITY;
                s[rt][tb][i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
        float p[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[4 * tb + i] = fast_exp2(s[rt][tb][i] - st.m[rt]);
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

// DEPTH: blocks requested ahead of the one being computed (DEPTH + 1 register
// sets rotate).  NTL: nontemporal K/V loads.  FUSED: the row's tokens continue
// past n_c in a second segment (the local block of a fused decode step).
template <int NT>
union SplitSmem {
    MfmaSmem<NT> m;
    char ring[kWaves][2][kSlotBytes];
};

template <int NT, int DEPTH, bool NTL, bool FUSED, bool RING>
__global__ __launch_bounds__(64 * kWaves) void k_split_mfma(SplitArgs a) {
    __shared__ __attribute__((aligned(16))) SplitSmem<NT> smu;
    MfmaSmem<NT>& sm = smu.m;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j = lane >> 4, c16 = lane & 15;
    const int split = blockIdx.x, h = blockIdx.y;
    const int bkv = blockIdx.z / a.row_groups, rg = blockIdx.z % a.row_groups;
    const int rows_base = rg * 16 * NT;

    int64_t n_eff = a.n;
    if (a.n_b) n_eff = min((int64_t)a.n_b[bkv], a.n);
    const int64_t head_off = (int64_t)bkv * a.kv_batch_stride + (int64_t)h * a.n * kD;
    Segs sg;
    sg.kh = static_cast<const uint16_t*>(a.k) + head_off;
    sg.vh = static_cast<const uint16_t*>(a.v) + head_off;
    sg.n_c = a.n;
    sg.kh2 = sg.vh2 = nullptr;
    if (FUSED) {
        const int64_t off2 = (int64_t)bkv * a.kv2_batch_stride + (int64_t)h * a.n2 * kD;
        sg.kh2 = static_cast<const uint16_t*>(a.k2) + off2;
        sg.vh2 = static_cast<const uint16_t*>(a.v2) + off2;
        n_eff = a.n + (a.n2_b ? min(max((int64_t)a.n2_b[bkv], (int64_t)0), a.n2) : a.n2);
    }

    const int64_t t_begin = (int64_t)split * a.blocks_per_split * kBlock;
    const int64_t t_end = min(n_eff, t_begin + (int64_t)a.blocks_per_split * kBlock);
    const int64_t step = (int64_t)kWaves * kBlock;
    const int64_t last = n_eff - 1;
    int64_t t = t_begin + w * kBlock;

    // Direct mode with a (alpha_in, a_in) pair: read the values this thread
    // will finish now, so their latency hides behind the main loop.
    constexpr int kFin = 16 * NT * kD / (64 * kWaves);
    float pre_al[kFin], pre_a[kFin];
    if (a.direct && a.alpha_in) {   // uniform; clamped rows keep the loads branch-free
#pragma unroll
        for (int f = 0; f < kFin; ++f) {
            const int e = threadIdx.x + f * 64 * kWaves;
            const int r = min(rows_base + e / kD, a.rows - 1);
            const int b = a.shared ? r / a.G : bkv;
            const int g = a.shared ? r % a.G : r;
            const int64_t bhq = (int64_t)b * a.Hq + h * a.G + g;
            pre_al[f] = a.alpha_in[bhq];
            pre_a[f] = a.a_in[bhq * kD + e % kD];
        }
    } else {
#pragma unroll
        for (int f = 0; f < kFin; ++f) {
            pre_al[f] = -INFINITY;
            pre_a[f] = 0.f;
        }
    }

    WaveState<NT> st;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        const int r = rows_base + rt * 16 + c16;
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

    if (RING) {
        // Drain the prologue's own loads, then request the first two blocks
        // into this wave's two slots.  Past the end of the range the current
        // block is requested again (cache-resident), which keeps exactly one
        // block's loads (16) younger than the block being waited for.
        wait_vm_all();
        char* slots = smu.ring[w][0];
        const uint32_t lane_off = lds_addr(slots) + 16 * lane;
        int slot = 0;
        if (t < t_end) {
            dma_block<NTL, FUSED>(slots, sg, t, last, j, c16);
            const int64_t t1 = t + step;
            dma_block<NTL, FUSED>(slots + kSlotBytes, sg, t1 < t_end ? t1 : t, last, j, c16);
            while (true) {
                __builtin_amdgcn_s_waitcnt(kVmcnt16);   // this slot has landed
                BlockRegs r;
                lds_read_block(r, lane_off + slot * kSlotBytes);
                const int64_t tn = t + 2 * step;
                dma_block<NTL, FUSED>(slots + slot * kSlotBytes, sg, tn < t_end ? tn : t, last, j, c16);
                compute_block<NT>(st, r, t, n_eff, a.scale_log2, j, c16);
                t += step;
                if (t >= t_end) break;
                slot ^= 1;
            }
        }
        wait_vm_all();     // the refills past the end
        __syncthreads();   // every wave is done with its slots before they become the merge buffer
    } else {
    // Request the first DEPTH blocks, then drain everything issued so far (the
    // query fragments, the merge inputs and these blocks), so that inside the
    // loop only the loop's own block loads are ever outstanding.  Past the end
    // of the range the current block is requested again (cache-resident),
    // which keeps the number of loads per step uniform.
    BlockRegs buf[DEPTH + 1];
    if (t < t_end) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int64_t tu = t + u * step;
            load_block<NTL, FUSED>(buf[u], sg, tu < t_end ? tu : t, last, j, c16);
        }
    }
    wait_vm_all();

    if (t < t_end) {
        bool done = false;
        while (!done) {
#pragma unroll
            for (int u = 0; u <= DEPTH; ++u) {
                if (!done) {
                    const int64_t tn = t + DEPTH * step;
                    load_block<NTL, FUSED>(buf[(u + DEPTH) % (DEPTH + 1)], sg, tn < t_end ? tn : t, last, j, c16);
                    // Keep every load of the block ahead above the first use of the current one.
                    __builtin_amdgcn_sched_barrier(0);
                    compute_block<NT>(st, buf[u], t, n_eff, a.scale_log2, j, c16);
                    t += step;
                    done = t >= t_end;
                }
            }
        }
    }
    }

    // Per-wave state -> LDS.
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        float l = st.l[rt];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (j == 0) sm.ml[w][rt * 16 + c16] = make_float2(st.m[rt], l);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float* dst = &sm.o[w][rt * 16 + 4 * j + i][8 * c16];
            *reinterpret_cast<f32x4*>(dst) = f32x4{st.o[rt][0][i], st.o[rt][1][i], st.o[rt][2][i], st.o[rt][3][i]};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{st.o[rt][4][i], st.o[rt][5][i], st.o[rt][6][i], st.o[rt][7][i]};
        }
    }
    __syncthreads();

    // Merge the waves' states; one slot per (row, split).
#pragma unroll
    for (int f = 0; f < kFin; ++f) {
        const int e = threadIdx.x + f * 64 * kWaves;
        const int row = e / kD, c = e % kD;
        const int r = rows_base + row;
        if (r >= a.rows) continue;
        float M = sm.ml[0][row].x;
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm.ml[ww][row].x);
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float wt = fast_exp2(sm.ml[ww][row].x - M);
            L += wt * sm.ml[ww][row].y;
            acc += wt * sm.o[ww][row][c];
        }
        const int b = a.shared ? r / a.G : bkv;
        const int g = a.shared ? r % a.G : r;
        const int64_t bhq = (int64_t)b * a.Hq + h * a.G + g;
        if (a.direct) {
            finish_row(a, bhq, c, M, L, acc, pre_al[f] > -INFINITY, pre_al[f], pre_a[f]);
        } else {
            const int64_t slot = bhq * a.splits + split;
            a.acc[slot * kD + c] = acc;
            if (c == 0) a.ml[slot] = make_float2(M, L);
        }
    }
}

}  // namespace

hipError_t launch_split_mfma(const SplitPlan& p, const SplitArgs& a, hipStream_t st) {
    dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(64 * kWaves);
    const int variant = (int)tuning().dense_variant;
    const bool fused = a.k2 != nullptr;
#define LCDA_SPLIT(NT_, NTL_, RING_)                                                                   \
    do {                                                                                               \
        if (fused) hipLaunchKernelGGL((k_split_mfma<NT_, 1, NTL_, true, RING_>), grid, block, 0, st, a); \
        else hipLaunchKernelGGL((k_split_mfma<NT_, 1, NTL_, false, RING_>), grid, block, 0, st, a);    \
    } while (0)
    switch (p.nt) {
        case 1:
            if (variant == 1) LCDA_SPLIT(1, false, false);
            else if (variant == 2) LCDA_SPLIT(1, true, true);
            else LCDA_SPLIT(1, true, false);
            break;
        case 2: LCDA_SPLIT(2, true, false); break;
        case 4: LCDA_SPLIT(4, true, false); break;
        default: return hipErrorInvalidValue;
    }
#undef LCDA_SPLIT
    return hipGetLastError();
}

}  // namespace lcda
