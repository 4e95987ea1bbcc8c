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
// - K/V blocks are read with buffer loads against a per-block resource (the
//   block's first row in scalar registers, its size the rows left in the
//   segment), so a lane holds two 32-bit offsets instead of 16 addresses, and
//   rows past the end read as zero; their scores are masked.
// - The next block's loads are issued before the current block is computed.
// - The 4 waves of a workgroup interleave blocks of the split and merge their
//   states through LDS, so each (row, split) slot is written once.

#include "common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace lcda {
namespace {

// A row's token range: segment 1 (kh, vh) holds rows [0, n_c); in a fused step
// segment 2 (kh2, vh2) holds its rows at unified tokens [n_c_al, n_eff), where
// n_c_al is n_c rounded up to a whole block, so no block spans both segments
// (the at most 31 positions in between are masked like a tail).
struct Segs {
    const uint16_t* kh;
    const uint16_t* vh;
    const uint16_t* kh2;
    const uint16_t* vh2;
    int64_t n_c, n_c_al, n_eff;
};


// Block of 32 tokens starting at unified token t: returns the rows of it that
// hold tokens (1..32) and requests all 32 rows; rows past the segment's end
// read as zero.  With live == false (a request past the end of the wave's
// range, issued so that every loop step has the same loads outstanding) the
// resource is empty: the loads return zeros and touch no memory.
// koff = 256*c16 + 16*j (K row c16 of each 16-token half); voff = 1024*j +
// 16*c16 (V row 4j): the V rows tok_of(j, e) are 4j + e and 16 + 4j + (e - 4).
template <bool NTL, bool FUSED>
__device__ __forceinline__ int load_block(BlockRegs& r, const Segs& sg, int64_t t, bool live, uint32_t koff,
                                          uint32_t voff) {
    const bool second = FUSED && t >= sg.n_c_al;
    const uint16_t* kseg = second ? sg.kh2 : sg.kh;
    const uint16_t* vseg = second ? sg.vh2 : sg.vh;
    const int64_t row = second ? t - sg.n_c_al : t;
    const int64_t left = (second ? sg.n_eff - sg.n_c_al : (FUSED ? sg.n_c : sg.n_eff)) - row;
    const int valid = (int)(left < kBlock ? left : kBlock);
    const int nrec = live ? valid * kD * 2 : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kseg + row * kD), 0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vseg + row * kD), 0, nrec, kRsrcWord3);
    constexpr int aux = NTL ? 2 : 0;   // nontemporal
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

// DEPTH: blocks requested ahead of the one being computed (DEPTH + 1 register
// sets rotate).  NTL: nontemporal K/V loads.  FUSED: the row's tokens continue
// in a second segment (the local block of a fused decode step).  WPE: waves
// per SIMD the register allocation leaves room for (2 caps a wave at 256
// VGPRs so two workgroups share a CU).  DIRECT: one split per unit, rows
// finished in place (a.direct).
template <int NT, int DEPTH, bool NTL, bool FUSED, int WPE, bool DIRECT>
__global__ __launch_bounds__(64 * kWaves, WPE) void k_split_mfma(SplitArgs a) {
    __shared__ __attribute__((aligned(16))) MfmaSmem<NT> sm;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: keeps t in scalars
    const int j = lane >> 4, c16 = lane & 15;
    const uint32_t koff = 256u * c16 + 16u * j;
    const uint32_t voff = 1024u * j + 16u * c16;
    const int split = blockIdx.x, h = blockIdx.y;
    const int bkv = blockIdx.z / a.row_groups, rg = blockIdx.z % a.row_groups;
    const int rows_base = rg * 16 * NT;

    const int64_t head_off = (int64_t)bkv * a.kv_batch_stride + (int64_t)h * a.n * kD;
    Segs sg;
    sg.kh = static_cast<const uint16_t*>(a.k) + head_off;
    sg.vh = static_cast<const uint16_t*>(a.v) + head_off;
    sg.n_c = a.n;
    sg.n_c_al = a.n;
    sg.kh2 = sg.vh2 = nullptr;
    sg.n_eff = a.n_b ? min((int64_t)a.n_b[bkv], a.n) : a.n;
    if (FUSED) {
        const int64_t off2 = (int64_t)bkv * a.kv2_batch_stride + (int64_t)h * a.n2 * kD;
        sg.kh2 = static_cast<const uint16_t*>(a.k2) + off2;
        sg.vh2 = static_cast<const uint16_t*>(a.v2) + off2;
        sg.n_c_al = (a.n + kBlock - 1) / kBlock * kBlock;
        sg.n_eff = sg.n_c_al + (a.n2_b ? min(max((int64_t)a.n2_b[bkv], (int64_t)0), a.n2) : a.n2);
    }

    const int64_t t_begin = (int64_t)split * a.blocks_per_split * kBlock;
    const int64_t t_end = min(sg.n_eff, t_begin + (int64_t)a.blocks_per_split * kBlock);
    const int64_t step = (int64_t)kWaves * kBlock;
    int64_t t = t_begin + w * kBlock;

    // Direct mode with a (alpha_in, a_in) pair: read the values this thread
    // will finish now, so their latency hides behind the main loop.
    constexpr int kFin = 16 * NT * kD / (64 * kWaves);
    float pre_al[kFin], pre_a[kFin];
    if (DIRECT && a.alpha_in) {   // uniform; clamped rows keep the loads branch-free
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

    // Request the first DEPTH blocks, then drain everything issued so far (the
    // query fragments, the merge inputs and these blocks), so that inside the
    // loop only the loop's own block loads are ever outstanding.  Past the end
    // of the range an empty request is issued (no memory is read), which keeps
    // the number of loads per step uniform.
    BlockRegs buf[DEPTH + 1];
    int valid[DEPTH + 1];
    if (t < t_end) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int64_t tu = t + u * step;
            valid[u] = load_block<NTL, FUSED>(buf[u], sg, tu < t_end ? tu : t, tu < t_end, koff, voff);
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
                    const int nx = (u + DEPTH) % (DEPTH + 1);
                    valid[nx] = load_block<NTL, FUSED>(buf[nx], sg, tn < t_end ? tn : t, tn < t_end, koff, voff);
                    // Keep every load of the block ahead above the first use of the current one.
                    __builtin_amdgcn_sched_barrier(0);
                    compute_block<NT>(st, buf[u], valid[u], a.scale_log2, j, c16);
                    t += step;
                    done = t >= t_end;
                }
            }
        }
    }

    // Per-wave state -> LDS.
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        float l = st.l[rt];
        l = sum_xor32(sum_xor16(l));
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
        if (DIRECT) {
            finish_row(a, bhq, c, M, L, acc, pre_al[f] > -INFINITY, pre_al[f], pre_a[f]);
        } else {
            const int64_t slot = bhq * a.splits + split;
            store_dev(a.acc + slot * kD + c, acc);
            if (c == 0) store_dev(a.ml + slot, make_float2(M, L));
        }
    }

    // The unit's last workgroup to finish merges every split of its rows.
    if constexpr (!DIRECT) {
        __shared__ int s_last;
        const int64_t unit = ((int64_t)bkv * a.Hkv + h) * a.row_groups + rg;
        if (arrive_last(a, unit, &s_last)) {
            const int nrows = min(16 * NT, a.rows - rows_base);
            for (int rr = w; rr < nrows; rr += kWaves) {
                const int r = rows_base + rr;
                const int b = a.shared ? r / a.G : bkv;
                const int g = a.shared ? r % a.G : r;
                combine_row(a, (int64_t)b * a.Hq + h * a.G + g, lane);
            }
        }
    }
}

}  // namespace

hipError_t launch_split_mfma(const SplitPlan& p, const SplitArgs& a, hipStream_t st) {
    dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(64 * kWaves);
    const int variant = (int)tuning().dense_variant;
    const bool fused = a.k2 != nullptr;
    const bool direct = a.direct != 0;
#define LCDA_SPLIT(NT_, DEPTH_, NTL_, WPE_)                                                                   \
    do {                                                                                                      \
        if (fused && direct)                                                                                  \
            hipLaunchKernelGGL((k_split_mfma<NT_, DEPTH_, NTL_, true, WPE_, true>), grid, block, 0, st, a);   \
        else if (fused)                                                                                       \
            hipLaunchKernelGGL((k_split_mfma<NT_, DEPTH_, NTL_, true, WPE_, false>), grid, block, 0, st, a);  \
        else if (direct)                                                                                      \
            hipLaunchKernelGGL((k_split_mfma<NT_, DEPTH_, NTL_, false, WPE_, true>), grid, block, 0, st, a);  \
        else                                                                                                  \
            hipLaunchKernelGGL((k_split_mfma<NT_, DEPTH_, NTL_, false, WPE_, false>), grid, block, 0, st, a); \
    } while (0)
    switch (p.nt) {
        case 1:
            if (variant == 1) LCDA_SPLIT(1, 1, false, 1);
            else if (variant == 2) LCDA_SPLIT(1, 2, true, 1);
            else if (variant == 3 && !direct) LCDA_SPLIT(1, 1, true, 2);
            else LCDA_SPLIT(1, 1, true, 1);
            break;
        case 2: LCDA_SPLIT(2, 1, true, 1); break;
        case 4: LCDA_SPLIT(4, 1, true, 1); break;
        default: return hipErrorInvalidValue;
    }
#undef LCDA_SPLIT
    return hipGetLastError();
}

}  // namespace lcda
