// combine.hip - exact log-sum-exp combination of partial softmax states.
//
// Splitting the softmax sum is exact ("Nectar: Neural Estimation of
// Cached-Token Attention via Regression", slide "The score makes exact local
// attention composable"): with M = max_c m_c,
//   L = sum_c l_c 2^(m_c - M),   A = sum_c acc_c 2^(m_c - M) / L,
//   alpha = (M + log2 L) * ln 2.
// An optional (alpha_in, A_in) pair per row enters as one more state with
// m = alpha_in * log2(e), l = 1, acc = A_in: the "virtual logit/value pair"
// of Eq. (3.4), which makes the same kernel the local-token merge.
//
// k_combine, for many slots: one workgroup of 256 threads per query row; the
// slot weights are computed once into LDS (maxima and sums reduced in each
// wavefront, then across the four through LDS), then 8 slot groups x 32
// threads x 4 columns read the partial vectors with independent 16-byte loads
// and are summed through LDS.  k_combine_small, for at most 64 slots: one
// wavefront per row.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = kThreads / 32;   // slot groups; 32 threads x float4 cover d = 128

__global__ __launch_bounds__(kThreads) void k_combine(CombineArgs a) {
    constexpr int kW = kThreads / 64;
    __shared__ float s_w[1024];
    __shared__ float s_red[2][kW];   // per-wavefront max, then per-wavefront sum
    __shared__ int s_anyw[kW];
    __shared__ f32x4 s_acc[kGroups][32];
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv_id = tid >> 6;
    const int S = a.slots;
    const float2* ml = a.ml + (int64_t)row * S;

    const float al_in = a.alpha_in != nullptr ? a.alpha_in[row] : -INFINITY;   // one load, requested first
    const bool virt = al_in > -INFINITY;
    const float mv = virt ? al_in * kLog2e : kNoMax;

    // Request the first kPre slots of each group's partial vectors before
    // anything else; the weights are computed while they are in flight.
    constexpr int kPre = 8;
    const int g = tid / 32, c4 = tid % 32;
    const float* acc = a.acc + (int64_t)row * S * kD + 4 * c4;
    f32x4 pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int s = g + kGroups * k;
        pre[k] = *reinterpret_cast<const f32x4*>(acc + (int64_t)min(s, S - 1) * kD);   // clamped; unused if s >= S
    }

    // M over non-empty slots (and the virtual pair).  A thread's first slot
    // state stays in registers for the weights below (with at most kThreads
    // slots it is the thread's only one).
    const float2 x0 = tid < S ? ml[tid] : make_float2(kNoMax, 0.f);
    float mloc = x0.y > 0.f ? x0.x : kNoMax;
    int anyloc = x0.y > 0.f ? 1 : 0;
    for (int s = tid + kThreads; s < S; s += kThreads) {
        const float2 x = ml[s];
        if (x.y > 0.f) {
            mloc = fmaxf(mloc, x.x);
            anyloc = 1;
        }
    }
    // Wavefront reductions, then one exchange of the kW wavefront values.
    mloc = wave_max(mloc);
    const bool anyw = __any(anyloc) != 0;
    if (lane == 0) {
        s_red[0][wv_id] = mloc;
        s_anyw[wv_id] = anyw ? 1 : 0;
    }
    __syncthreads();
    float Mw = s_red[0][0];
    int anyall = s_anyw[0];
#pragma unroll
    for (int k = 1; k < kW; ++k) {
        Mw = fmaxf(Mw, s_red[0][k]);
        anyall |= s_anyw[k];
    }
    const bool any = anyall != 0 || virt;
    const float M = fmaxf(Mw, virt ? mv : kNoMax);
    if (!any) {
        if (tid < kD) a.out[(int64_t)row * kD + tid] = 0.f;
        if (a.alpha && tid == 0) a.alpha[row] = -INFINITY;
        return;
    }
    // Slot weights w_s = 2^(m_s - M) (0 for empty slots) and L.
    float lloc = 0.f;
    if (tid < S) {
        const float w = x0.y > 0.f ? fast_exp2(x0.x - M) : 0.f;
        if (tid < 1024) s_w[tid] = w;
        lloc = w * x0.y;
    }
    for (int s = tid + kThreads; s < S; s += kThreads) {
        const float2 x = ml[s];
        const float w = x.y > 0.f ? fast_exp2(x.x - M) : 0.f;
        if (s < 1024) s_w[s] = w;
        lloc += w * x.y;
    }
    lloc = wave_sum(lloc);
    if (lane == 0) s_red[1][wv_id] = lloc;
    __syncthreads();   // also publishes s_w
    float Ls = 0.f;
#pragma unroll
    for (int k = 0; k < kW; ++k) Ls += s_red[1][k];
    const float wv = virt ? fast_exp2(mv - M) : 0.f;
    const float L = Ls + wv;

    // Weighted sum of the partial vectors: thread (group g, lane c4) owns columns 4*c4..4*c4+3.
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int s = g + kGroups * k;
        if (s < S) x += (s < 1024 ? s_w[s] : (ml[s].y > 0.f ? fast_exp2(ml[s].x - M) : 0.f)) * pre[k];
    }
#pragma unroll 4
    for (int s = g + kGroups * kPre; s < S; s += kGroups) {
        const float w = s < 1024 ? s_w[s] : (ml[s].y > 0.f ? fast_exp2(ml[s].x - M) : 0.f);
        const f32x4 v = *reinterpret_cast<const f32x4*>(acc + (int64_t)s * kD);
        x += w * v;
    }
    s_acc[g][c4] = x;
    __syncthreads();
    if (tid < 32) {
        f32x4 t = s_acc[0][tid];
#pragma unroll
        for (int gg = 1; gg < kGroups; ++gg) t += s_acc[gg][tid];
        if (virt) t += wv * *reinterpret_cast<const f32x4*>(a.a_in + (int64_t)row * kD + 4 * tid);
        const float inv = 1.f / L;
        *reinterpret_cast<f32x4*>(a.out + (int64_t)row * kD + 4 * tid) = t * inv;
        if (a.alpha && tid == 0) a.alpha[row] = (M + log2f(L)) * kLn2;
    }
}

// Rows of at most SM slots (1 <= slots <= SM): one wavefront per row, four
// rows per workgroup.  Every load of a row is requested at once (the slot
// states one per lane, the partial vectors of all slots, two columns per
// lane), so the merge waits for one memory round trip; then the same
// arithmetic as above, the slots summed in order.
template <int SM>
__global__ __launch_bounds__(kThreads) void k_combine_small(CombineArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= a.rows) return;   // a whole wavefront; no barrier follows
    const int S = a.slots;
    const float2 x = a.ml[row * S + min(lane, S - 1)];   // lanes at or past S are ignored
    const float* acc = a.acc + row * S * kD + 2 * lane;
    f32x2 v[SM];
#pragma unroll
    for (int s = 0; s < SM; ++s) v[s] = *reinterpret_cast<const f32x2*>(acc + (int64_t)min(s, S - 1) * kD);
    const float al_in = a.alpha_in != nullptr ? a.alpha_in[row] : -INFINITY;
    const bool virt = al_in > -INFINITY;
    const f32x2 a_in = virt ? *reinterpret_cast<const f32x2*>(a.a_in + row * kD + 2 * lane) : f32x2{0.f, 0.f};
    const bool has = lane < S && x.y > 0.f;
    if (!__any(has) && !virt) {
        *reinterpret_cast<f32x2*>(a.out + row * kD + 2 * lane) = f32x2{0.f, 0.f};
        if (a.alpha && lane == 0) a.alpha[row] = -INFINITY;
        return;
    }
    const float mv = virt ? al_in * kLog2e : kNoMax;
    const float M = fmaxf(wave_max(has ? x.x : kNoMax), mv);
    const float w = has ? fast_exp2(x.x - M) : 0.f;
    f32x2 o = {0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SM; ++s)
        if (s < S) o += __shfl(w, s, 64) * v[s];   // s < S is the same in every lane
    const float wv = virt ? fast_exp2(mv - M) : 0.f;
    const float L = wave_sum(w * x.y) + wv;
    if (virt) o += wv * a_in;
    *reinterpret_cast<f32x2*>(a.out + row * kD + 2 * lane) = o * (1.f / L);
    if (a.alpha && lane == 0) a.alpha[row] = (M + log2f(L)) * kLn2;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    if (a.rows <= 0) return hipSuccess;
    if (a.slots >= 1 && a.slots <= 64) {   // few slots per row: a wavefront per row
        const dim3 grid((unsigned)((a.rows + kThreads / 64 - 1) / (kThreads / 64)));
        if (a.slots <= 4) hipLaunchKernelGGL(k_combine_small<4>, grid, dim3(kThreads), 0, st, a);
        else if (a.slots <= 8) hipLaunchKernelGGL(k_combine_small<8>, grid, dim3(kThreads), 0, st, a);
        else if (a.slots <= 16) hipLaunchKernelGGL(k_combine_small<16>, grid, dim3(kThreads), 0, st, a);
        else if (a.slots <= 32) hipLaunchKernelGGL(k_combine_small<32>, grid, dim3(kThreads), 0, st, a);
        else hipLaunchKernelGGL(k_combine_small<64>, grid, dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_combine, dim3(a.rows), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcda
