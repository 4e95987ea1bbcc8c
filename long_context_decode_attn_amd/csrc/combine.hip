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
// One workgroup of 256 threads per query row: the slot weights are computed
// once into LDS, then 8 slot groups x 32 threads x 4 columns read the partial
// vectors with independent 16-byte loads and are summed through LDS.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = kThreads / 32;   // slot groups; 32 threads x float4 cover d = 128

__global__ __launch_bounds__(kThreads) void k_combine(CombineArgs a) {
    __shared__ float s_w[1024];
    __shared__ float s_red[kThreads];
    __shared__ f32x4 s_acc[kGroups][32];
    __shared__ float s_M, s_L;
    __shared__ int s_any;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int S = a.slots;
    const float2* ml = a.ml + (int64_t)row * S;

    const bool virt = a.alpha_in != nullptr && a.alpha_in[row] > -INFINITY;
    const float mv = virt ? a.alpha_in[row] * kLog2e : kNoMax;

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

    // M over non-empty slots (and the virtual pair).
    float mloc = kNoMax;
    int anyloc = 0;
    for (int s = tid; s < S; s += kThreads) {
        const float2 x = ml[s];
        if (x.y > 0.f) {
            mloc = fmaxf(mloc, x.x);
            anyloc = 1;
        }
    }
    s_red[tid] = mloc;
    if (tid == 0) s_any = 0;
    __syncthreads();
    if (anyloc) s_any = 1;
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (tid < o) s_red[tid] = fmaxf(s_red[tid], s_red[tid + o]);
        __syncthreads();
    }
    const bool any = s_any || virt;
    const float M = fmaxf(s_red[0], virt ? mv : kNoMax);
    __syncthreads();
    if (!any) {
        if (tid < kD) a.out[(int64_t)row * kD + tid] = 0.f;
        if (a.alpha && tid == 0) a.alpha[row] = -INFINITY;
        return;
    }
    // Slot weights w_s = 2^(m_s - M) (0 for empty slots) and L.
    float lloc = 0.f;
    for (int s = tid; s < S; s += kThreads) {
        const float2 x = ml[s];
        const float w = x.y > 0.f ? fast_exp2(x.x - M) : 0.f;
        if (s < 1024) s_w[s] = w;
        lloc += w * x.y;
    }
    s_red[tid] = lloc;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (tid < o) s_red[tid] += s_red[tid + o];
        __syncthreads();
    }
    const float wv = virt ? fast_exp2(mv - M) : 0.f;
    const float L = s_red[0] + wv;

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

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    if (a.rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_combine, dim3(a.rows), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcda
