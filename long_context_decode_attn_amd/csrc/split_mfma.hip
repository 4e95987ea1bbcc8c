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

__device__ __forceinline__ void load_block(BlockRegs& r, const uint16_t* kh, const uint16_t* vh,
                                           int64_t t, int64_t last, int j, int c16) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int64_t tok = min(t + 16 * tb + c16, last);
        const uint16_t* p = kh + tok * kD + 8 * j;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.k[tb][c] = ld16(p + 32 * c);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t tok = min(t + tok_of(j, e), last);
        r.v[e] = ld16(vh + tok * kD + 8 * c16);
    }
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

template <int NT>
__global__ __launch_bounds__(64 * kWaves) void k_split_mfma(SplitArgs a) {
    __shared__ MfmaSmem<NT> sm;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j = lane >> 4, c16 = lane & 15;
    const int split = blockIdx.x, h = blockIdx.y;
    const int bkv = blockIdx.z / a.row_groups, rg = blockIdx.z % a.row_groups;
    const int rows_base = rg * 16 * NT;

    int64_t n_eff = a.n;
    if (a.n_b) n_eff = min((int64_t)a.n_b[bkv], a.n);
    const int64_t head_off = (int64_t)bkv * a.kv_batch_stride + (int64_t)h * a.n * kD;
    const uint16_t* kh = static_cast<const uint16_t*>(a.k) + head_off;
    const uint16_t* vh = static_cast<const uint16_t*>(a.v) + head_off;

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

    const int64_t t_begin = (int64_t)split * a.blocks_per_split * kBlock;
    const int64_t t_end = min(n_eff, t_begin + (int64_t)a.blocks_per_split * kBlock);
    const int64_t step = (int64_t)kWaves * kBlock;
    const int64_t last = n_eff - 1;

    int64_t t = t_begin + w * kBlock;
    if (t < t_end) {
        // Two register sets; the next block is requested before the current one
        // is computed.  Past the end, the current block is requested again
        // (cache-resident), which keeps the load count uniform.
        BlockRegs ra, rb;
        load_block(ra, kh, vh, t, last, j, c16);
        while (true) {
            int64_t tn = t + step;
            load_block(rb, kh, vh, tn < t_end ? tn : t, last, j, c16);
            compute_block<NT>(st, ra, t, n_eff, a.scale_log2, j, c16);
            t = tn;
            if (t >= t_end) break;
            tn = t + step;
            load_block(ra, kh, vh, tn < t_end ? tn : t, last, j, c16);
            compute_block<NT>(st, rb, t, n_eff, a.scale_log2, j, c16);
            t = tn;
            if (t >= t_end) break;
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
    for (int e = threadIdx.x; e < 16 * NT * kD; e += 64 * kWaves) {
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
        const int64_t slot = ((int64_t)b * a.Hq + h * a.G + g) * a.splits + split;
        a.acc[slot * kD + c] = acc;
        if (c == 0) a.ml[slot] = make_float2(M, L);
    }
}

}  // namespace

hipError_t launch_split_mfma(const SplitPlan& p, const SplitArgs& a, hipStream_t st) {
    dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(64 * kWaves);
    switch (p.nt) {
        case 1: hipLaunchKernelGGL(k_split_mfma<1>, grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL(k_split_mfma<2>, grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL(k_split_mfma<4>, grid, block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lcda
