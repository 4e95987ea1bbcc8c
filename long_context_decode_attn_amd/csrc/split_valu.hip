// split_valu.hip - split attention partials on the vector ALUs, for fp32 or
// bf16 K/V, over a token range (dense) or over a list of selected positions
// (GATHER-ATT of "HashAttention: Semantic Sparsity for Faster Inference",
// slide "Only selection is approximate; selected KV stay in full form":
// softmax renormalised over the selected set, rows read straight from the
// cache by position, page size 1, no gathered copy).
//
// Partial state per row and slot as in split_mfma.hip (base-2 units), merged
// by the combine pass.
//
// Mapping: 16 lanes share one K/V row, each lane holding 8 consecutive d
// values (16 B for bf16, 32 B for fp32), so one load instruction reads 4 whole
// rows; the 4 lane groups of a wave walk interleaved token subsequences, each
// with its own online softmax, and are merged by cross-lane shuffles at the
// end.  Dot products are reduced over the 16 lanes of a row by butterflies.
// Each lane group takes U rows per step and rescales once per step.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

constexpr int kWaves = 4;

template <typename T>
struct Row8;

template <>
struct Row8<float> {
    u32x4 a, b;
    template <bool NT = false>
    __device__ __forceinline__ void load(const float* p) {
        a = ld16s<NT>(p);
        b = ld16s<NT>(p + 4);
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
struct Row8<uint16_t> {
    u32x4 a;
    template <bool NT = false>
    __device__ __forceinline__ void load(const uint16_t* p) { a = ld16s<NT>(p); }
    __device__ __forceinline__ void to_float(float (&x)[8]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(a[e]);
            x[2 * e + 1] = bf16_hi(a[e]);
        }
    }
};

template <typename T, int R, int W>
struct ValuSmem {
    float o[W][R][kD];
    float2 ml[W][R];
};

// R: query rows per unit (dense) - 1 in gather mode.  U: rows per lane group per step.
// NTL: K/V rows are loaded nontemporal.  W: wavefronts per workgroup, which
// share the split's token range step by step.  RA: steps whose rows are in
// flight ahead of the step computed (positions one step further).
template <typename T, int R, int U, bool GATHER, bool NTL, int W = kWaves, int RA = 2>
__global__ __launch_bounds__(64 * W) void k_split_valu(SplitArgs a) {
    __shared__ ValuSmem<T, R, W> sm;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int j = lane >> 4, c16 = lane & 15;
    const int split = blockIdx.x;
    constexpr int kStep = 4 * U;  // tokens per wave step

    // Unit: dense (bkv, h, rg) over grid (split, h, bkv*row_groups + rg);
    //       gather (b, hq) over grid (split, hq, b).
    int bkv, h, rows_base, n_rows;
    int64_t n_tok;
    const int32_t* list = nullptr;
    if (GATHER) {
        // blockIdx.y walks the KV heads fastest, so that the G query heads of
        // one KV head sit Hkv workgroups apart in dispatch order: on the same
        // XCD (workgroups go round the 8 XCDs in turn) when Hkv * splits is a
        // multiple of 8, where the rows the heads share hit that XCD's L2.
        const int hq = (int)(blockIdx.y % a.Hkv) * a.G + (int)(blockIdx.y / a.Hkv), b = blockIdx.z;
        h = hq / a.G;
        bkv = a.shared ? 0 : b;
        rows_base = 0;
        n_rows = 1;
        // Counts and positions are clamped to the buffers, so entries outside
        // the documented ranges give undefined values but never a stray access.
        n_tok = min(max((int64_t)a.count[(int64_t)b * a.Hq + hq], (int64_t)0), a.cap);
        list = a.idx + ((int64_t)b * a.Hq + hq) * a.cap;
    } else {
        h = blockIdx.y;
        bkv = blockIdx.z / a.row_groups;
        rows_base = (blockIdx.z % a.row_groups) * R;
        n_rows = min(R, a.rows - rows_base);
        n_tok = a.n;
        if (a.n_b) n_tok = min((int64_t)a.n_b[bkv], a.n);
    }
    const int64_t head_off = (int64_t)bkv * a.kv_batch_stride + (int64_t)h * a.n * kD;
    const T* kh = static_cast<const T*>(a.k) + head_off + 8 * c16;
    const T* vh = static_cast<const T*>(a.v) + head_off + 8 * c16;

    // Query rows of this unit -> (b, hq).
    auto row_bhq = [&](int r, int& b, int& hq) {
        if (GATHER) {
            b = blockIdx.z;
            hq = (int)(blockIdx.y % a.Hkv) * a.G + (int)(blockIdx.y / a.Hkv);
        } else {
            const int rr = rows_base + r;
            b = a.shared ? rr / a.G : bkv;
            hq = h * a.G + (a.shared ? rr % a.G : rr);
        }
    };

    float qv[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < n_rows) {
            int b, hq;
            row_bhq(r, b, hq);
            Row8<T> x;
            x.load(static_cast<const T*>(a.q) + ((int64_t)b * a.Hq + hq) * kD + 8 * c16);
            x.to_float(qv[r]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[r][e] = 0.f;
        }
    }

    // Direct mode with a (alpha_in, a_in) pair: read the values this thread
    // will finish now, so their latency hides behind the main loop.
    constexpr int kFin = (R * kD + 64 * W - 1) / (64 * W);
    float pre_al[kFin], pre_a[kFin];
#pragma unroll
    for (int f = 0; f < kFin; ++f) {
        pre_al[f] = -INFINITY;
        pre_a[f] = 0.f;
        const int e = threadIdx.x + f * 64 * W;
        const int r = e / kD;
        if (a.direct && a.alpha_in && e < R * kD && r < n_rows) {
            int b, hq;
            row_bhq(r, b, hq);
            const int64_t bhq = (int64_t)b * a.Hq + hq;
            pre_al[f] = a.alpha_in[bhq];
            pre_a[f] = a.a_in[bhq * kD + e % kD];
        }
    }

    float m[R], l[R], acc[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m[r] = kNoMax;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    }

    const int64_t t_begin = (int64_t)split * a.blocks_per_split * kStep;
    const int64_t t_end = min(n_tok, t_begin + (int64_t)a.blocks_per_split * kStep);
    const int64_t stride = (int64_t)W * kStep;

    // Software pipeline over steps of kStep tokens: the positions (gather mode:
    // entries of the index list) are requested RA + 1 steps ahead and the K/V
    // rows RA steps ahead of the step being computed.  Requests past the end
    // of the range are clamped to its last entry (cache-resident) and ignored.
    struct Step {
        Row8<T> k[U], v[U];
    };
    auto positions = [&](int64_t t0, int32_t (&pos)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = min(t0 + 4 * u + j, t_end - 1);
            pos[u] = GATHER ? min(max(list[t], 0), (int32_t)(a.n - 1)) : (int32_t)t;
        }
    };
    auto fetch = [&](Step& st, const int32_t (&pos)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            st.k[u].template load<NTL>(kh + (int64_t)pos[u] * kD);
            st.v[u].template load<NTL>(vh + (int64_t)pos[u] * kD);
        }
    };
    auto compute = [&](const Step& stp, int64_t t0) {
        float s[U][R];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[8];
            stp.k[u].to_float(kf);
            const bool valid = t0 + 4 * u + j < t_end;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qv[r][e], kf[e], d);
                d = sum16(d) * a.scale_log2;
                s[u][r] = valid ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float bm = s[0][r];
#pragma unroll
            for (int u = 1; u < U; ++u) bm = fmaxf(bm, s[u][r]);
            const float mnew = fmaxf(m[r], bm);
            const float alpha = fast_exp2(m[r] - mnew);
            m[r] = mnew;
            l[r] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[8];
            stp.v[u].to_float(vf);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float p = fast_exp2(s[u][r] - m[r]);
                l[r] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(p, vf[e], acc[r][e]);
            }
        }
    };

    // Step i of this wavefront lives in slot i mod NS of the buffers: at step
    // i the positions of step i + NS replace its own (fetched RA steps ago),
    // the rows of step i + RA are requested, and step i is computed.
    int64_t t0 = t_begin + (int64_t)w * kStep;
    if (t0 < t_end) {
        constexpr int NS = RA + 1;
        int32_t pp[NS][U];
        Step ss[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) positions(t0 + k * stride, pp[k]);
#pragma unroll
        for (int k = 0; k < RA; ++k) fetch(ss[k], pp[k]);
        bool done = false;
        while (!done) {
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                if (!done) {
                    positions(t0 + NS * stride, pp[u]);
                    fetch(ss[(u + RA) % NS], pp[(u + RA) % NS]);
                    compute(ss[u], t0);
                    t0 += stride;
                    done = t0 >= t_end;
                }
            }
        }
    }

    // Merge the 4 lane groups of the wave (lanes c16, c16+16, c16+32, c16+48).
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float M = max_xor32(max_xor16(m[r]));
        const float wt = fast_exp2(m[r] - M);
        const float L = sum_xor32(sum_xor16(l[r] * wt));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = sum_xor32(sum_xor16(acc[r][e] * wt));
        if (j == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.o[w][r][8 * c16 + e] = acc[r][e];
            if (c16 == 0) sm.ml[w][r] = make_float2(M, L);
        }
    }
    __syncthreads();

#pragma unroll
    for (int f = 0; f < kFin; ++f) {
        const int e = threadIdx.x + f * 64 * W;
        const int r = e / kD, c = e % kD;
        if (e >= R * kD || r >= n_rows) continue;
        float M = sm.ml[0][r].x;
#pragma unroll
        for (int ww = 1; ww < W; ++ww) M = fmaxf(M, sm.ml[ww][r].x);
        float L = 0.f, x = 0.f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) {
            const float wt = fast_exp2(sm.ml[ww][r].x - M);
            L += wt * sm.ml[ww][r].y;
            x += wt * sm.o[ww][r][c];
        }
        int b, hq;
        row_bhq(r, b, hq);
        const int64_t bhq = (int64_t)b * a.Hq + hq;
        if (a.direct) {
            finish_row(a, bhq, c, M, L, x, pre_al[f] > -INFINITY, pre_al[f], pre_a[f]);
        } else {
            const int64_t slot = bhq * a.splits + split;
            a.acc[slot * kD + c] = x;
            if (c == 0) a.ml[slot] = make_float2(M, L);
        }
    }
}

template <typename T, bool GATHER>
hipError_t launch_t(const SplitPlan& p, const SplitArgs& a, hipStream_t st) {
    dim3 grid(p.grid_x, p.grid_y, p.grid_z), block(64 * kWaves);
    constexpr int U = 4;
    if (GATHER) {
        const dim3 gblock(64 * p.waves);
        // 16 wavefronts (1,024 threads) leave 128 VGPRs a lane: rows one step ahead instead of two fit them.
        if (p.waves == 16) hipLaunchKernelGGL((k_split_valu<T, 1, U, true, true, 16, 1>), grid, gblock, 0, st, a);
        else if (p.waves == 8) {
            // fp32 rows take twice the registers: at 8 wavefronts (256 VGPRs a lane) rows two steps ahead
            // spilled one VGPR, so they go one step ahead.
            if constexpr (sizeof(T) == 4)
                hipLaunchKernelGGL((k_split_valu<T, 1, U, true, true, 8, 1>), grid, gblock, 0, st, a);
            else
                hipLaunchKernelGGL((k_split_valu<T, 1, U, true, true, 8>), grid, gblock, 0, st, a);
        }
        else if (tuning().gather_variant == 1) hipLaunchKernelGGL((k_split_valu<T, 1, U, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_split_valu<T, 1, U, true, true>), grid, block, 0, st, a);
    } else {
        switch (p.rows_per_group) {
            case 1: hipLaunchKernelGGL((k_split_valu<T, 1, U, false, false>), grid, block, 0, st, a); break;
            case 2: hipLaunchKernelGGL((k_split_valu<T, 2, U, false, false>), grid, block, 0, st, a); break;
            case 4: hipLaunchKernelGGL((k_split_valu<T, 4, U, false, false>), grid, block, 0, st, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace

int valu_step_tokens() { return 4 * 4; }

hipError_t launch_split_valu(const SplitPlan& p, const SplitArgs& a, int dtype, bool gather, hipStream_t st) {
    if (dtype == 0) return gather ? launch_t<float, true>(p, a, st) : launch_t<float, false>(p, a, st);
    return gather ? launch_t<uint16_t, true>(p, a, st) : launch_t<uint16_t, false>(p, a, st);
}

}  // namespace lcda
