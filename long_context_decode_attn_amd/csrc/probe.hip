// probe.hip - a plain streaming read of a device buffer, the measured ceiling
// against which the kernels' HBM rates are read (the published 8 TB/s is the
// interface's peak, not what a read kernel reaches).  Not part of the method.
//
// Each workgroup reads one contiguous share of the buffer (as a split-KV pass
// reads its token range), 64 KB per round: thread t loads 16-byte words
// t, t + 512, ... t + 7 x 512 of the round, nontemporal, the next round's loads
// issued before the current round is folded (so that 16 loads per thread are
// in flight), and folds what it reads into one word; the word is stored only
// if it equals a value the caller passes (so the loads cannot be removed, and
// nothing is written in practice).

#include "../../include/lcda.h"
#include "common.h"
#include "internal.h"

namespace lcda {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 8;

__device__ __forceinline__ uint32_t fold(const u32x4 (&x)[kProbeUnroll]) {
    uint32_t a = 0;
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) a ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
    return a;
}

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const u32x4* __restrict__ p, int64_t n16,
                                                               uint32_t* sink, uint32_t never) {
    constexpr int64_t kRound = (int64_t)kProbeUnroll * kProbeThreads;   // words per round
    // This workgroup's share [beg, end): whole rounds, the last share takes the rest.
    const int64_t rounds = (n16 + kRound - 1) / kRound;
    const int64_t per = (rounds + gridDim.x - 1) / gridDim.x;
    const int64_t beg = min(n16, (int64_t)blockIdx.x * per * kRound), end = min(n16, beg + per * kRound);
    const int64_t full_end = beg + (end - beg) / kRound * kRound;   // end of the whole rounds
    int64_t i = beg + threadIdx.x;
    uint32_t acc = 0;
    if (beg < full_end) {
        u32x4 a[kProbeUnroll], b[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) a[u] = ld16_nt(p + i + u * kProbeThreads);
        while (true) {
            const int64_t j = i + kRound;
            if (j >= full_end) {
                acc ^= fold(a);
                i = j;
                break;
            }
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) b[u] = ld16_nt(p + j + u * kProbeThreads);
            acc ^= fold(a);
            i = j + kRound;
            if (i >= full_end) {
                acc ^= fold(b);
                break;
            }
#pragma unroll
            for (int u = 0; u < kProbeUnroll; ++u) a[u] = ld16_nt(p + i + u * kProbeThreads);
            acc ^= fold(b);
        }
    }
    for (; i < end; i += kProbeThreads) {   // the part round of the last share
        const u32x4 x = ld16_nt(p + i);
        acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
    if (acc == never) sink[0] = acc;
}

}  // namespace
}  // namespace lcda

extern "C" int lcda_stream_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, uint32_t never,
                                void* stream) {
    static const char* fn = "lcda_stream_read";
    if (bytes == 0) return LCDA_OK;
    if (!buf || (reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15))
        return lcda::set_error(LCDA_EINVAL, "%s: buf must be non-null and 16-byte aligned, bytes a multiple of 16",
                               fn);
    if (!sink) return lcda::set_error(LCDA_EINVAL, "%s: sink is NULL", fn);
    if (workgroups <= 0 || workgroups > (1 << 20))
        return lcda::set_error(LCDA_EINVAL, "%s: workgroups = %d out of range", fn, workgroups);
    hipLaunchKernelGGL(lcda::k_stream_read, dim3((unsigned)workgroups), dim3(lcda::kProbeThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const lcda::u32x4*>(buf),
                       (int64_t)(bytes / 16), sink, never);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return lcda::set_error(LCDA_EHIP, "%s: %s", fn, hipGetErrorString(e));
    return LCDA_OK;
}
