// sig_encode.hip - T_map with a random projection: the 32-bit code of a
// 128-value row x has bit b = 1 when x . R[:, b] > 0 ("HashAttention: Semantic
// Sparsity for Faster Inference", slide "A 32-bit signature makes scoring
// cheap", Eq. (1), phi(x) = ReLU(sign(F(x))) with F(x) = R^T x: the
// random-projection selector of slide "Learning the codes matters more than
// merely hashing"; the learned map needs trained weights).
//
// Each projection is a chain of fp64 fused multiply-adds over the 128 values in
// order, from 0.  A bf16 or fp32 value times an fp32 value is exact in fp64 and
// the chain fixes the rounding of the sum, so every code, including the sign of
// a projection near zero, is reproducible bit for bit.
//
// A wavefront encodes two rows: lane l computes bit l % 32 of row 2w + l / 32.
// R sits in LDS as [128][32] fp32 (lanes l and l + 32 read the same word, the
// 32 lanes of a half read 32 consecutive words); every lane of a half reads the
// same 16 bytes of its row at a time; one ballot packs the 64 bits into the two
// rows' codes.

#include "common.h"
#include "internal.h"
#include "sparse.h"
#include "sig_proj.h"

namespace lcda {
namespace {

constexpr int kEncWaves = 4;
constexpr int kRowsPerWg = 2 * kEncWaves;

template <typename T>
__global__ __launch_bounds__(64 * kEncWaves) void k_sig_encode(EncodeArgs a) {
    __shared__ float sr[kD * 32];
    for (int k = threadIdx.x; k < kD * 32; k += 64 * kEncWaves) {
        const int e = k / 32, b = k % 32;
        sr[k] = b < a.bits ? a.R[e * a.bits + b] : 0.f;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t rows = a.groups * a.rows_per_group;
    const int64_t r = (int64_t)blockIdx.x * kRowsPerWg + 2 * w + (lane >> 5);
    const int64_t rr = min(r, rows - 1);   // a missing second row encodes the last one again, unused
    const int64_t g = rr / a.rows_per_group, i = rr % a.rows_per_group;
    const T* row = static_cast<const T*>(a.x) + g * a.x_group_stride + i * kD;
    float xf[kD];
    load_row(row, xf);
    const double z = proj_chain([&](int e) { return xf[e]; }, sr + (lane & 31), 32);
    const uint64_t bits = __ballot(z > 0.0);
    if ((lane & 31) == 0 && r < rows)
        a.codes[g * a.codes_group_stride + i] = (uint32_t)(lane == 0 ? bits : bits >> 32);
}

}  // namespace

hipError_t launch_sig_encode(const EncodeArgs& a, hipStream_t st) {
    const int64_t rows = a.groups * a.rows_per_group;
    if (rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg)), block(64 * kEncWaves);
    if (a.bf16) hipLaunchKernelGGL(k_sig_encode<uint16_t>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(k_sig_encode<float>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace lcda
