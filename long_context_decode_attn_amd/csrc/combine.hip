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
// One workgroup of 128 threads per query row, one thread per d column.

#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

__global__ __launch_bounds__(kD) void k_combine(CombineArgs a) {
    const int row = blockIdx.x;
    const int c = threadIdx.x;
    const float2* ml = a.ml + (int64_t)row * a.slots;
    const float* acc = a.acc + (int64_t)row * a.slots * kD + c;

    const bool virt = a.alpha_in != nullptr && a.alpha_in[row] > -INFINITY;
    const float mv = virt ? a.alpha_in[row] * kLog2e : kNoMax;

    float M = virt ? mv : kNoMax;
    bool any = virt;
    for (int s = 0; s < a.slots; ++s) {
        const float2 x = ml[s];
        if (x.y > 0.f) {
            M = fmaxf(M, x.x);
            any = true;
        }
    }
    float* out = a.out + (int64_t)row * kD + c;
    if (!any) {
        *out = 0.f;
        if (a.alpha && c == 0) a.alpha[row] = -INFINITY;
        return;
    }
    float L = 0.f, x = 0.f;
    if (virt) {
        const float wt = fast_exp2(mv - M);
        L = wt;
        x = wt * a.a_in[(int64_t)row * kD + c];
    }
    for (int s = 0; s < a.slots; ++s) {
        const float2 st = ml[s];
        if (st.y > 0.f) {
            const float wt = fast_exp2(st.x - M);
            L += wt * st.y;
            x += wt * acc[(int64_t)s * kD];
        }
    }
    *out = x / L;
    if (a.alpha && c == 0) a.alpha[row] = (M + log2f(L)) * kLn2;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
    if (a.rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_combine, dim3(a.rows), dim3(kD), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcda
