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
// Few rows (a step's queries, the new keys): a wavefront encodes two rows, lane
// l computing bit l % 32 of row 2w + l / 32.  R sits in LDS as [128][32] fp32
// (lanes l and l + 32 read the same word, the 32 lanes of a half read 32
// consecutive words); every lane of a half reads the same 16 bytes of its row
// at a time; one ballot packs the 64 bits into the two rows' codes.  This is
// the short path: one round of loads, then 128 dependent multiply-adds.
//
// Many rows (a whole cache): the work is 4,096 fp64 multiply-adds per row
// against 256 or 512 bytes read, so the fp64 issue rate bounds it.  Persistent
// workgroups of four wavefronts stage R once, already in fp64 ([128][32], 32 KB
// of LDS), and take 256 rows a turn.  Wave w computes bits 8w .. 8w + 7 of every
// row, so its projection values are the same for all its lanes (broadcast LDS
// reads); lane l owns rows 4l .. 4l + 3, 32 independent chains, each still in
// order from 0.  The rows come through LDS in 64-byte chunks stored
// [dword][row]: the global reads take whole 64-byte pieces of each row (a lane
// reading its own rows a few bytes at a time would make the L2 deliver a cache
// line per few bytes used), and a lane then reads its four rows' dword with one
// 16-byte LDS read.  The next chunk loads while this one is computed.  The four
// waves OR their bytes into the turn's codes in LDS.

#include <atomic>

#include "common.h"
#include "device.h"
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

constexpr int kManyP = 4;                   // rows per lane
constexpr int kManyRows = 64 * kManyP;      // rows per workgroup turn
constexpr int kManyXs = kManyRows + 4;      // dwords per LDS row of a staged chunk (padded)
constexpr int64_t kManyMinRows = 16384;     // below this the short path's latency wins

template <typename T>
__global__ __launch_bounds__(256, 2) void k_sig_encode_many(EncodeArgs a) {
    // R in fp64; a chunk of 64 bytes of each of the turn's rows as [dword][row]; the turn's codes.
    __shared__ double sr[kD * 32];
    __shared__ __align__(16) uint32_t xs[16 * kManyXs];
    __shared__ uint32_t cs[kManyRows];
    for (int k = threadIdx.x; k < kD * 32; k += 256) {
        const int e = k / 32, b = k % 32;
        sr[k] = b < a.bits ? (double)a.R[e * a.bits + b] : 0.0;
    }
    constexpr int kPer = 4 / sizeof(T);                  // values per dword
    constexpr int kChunks = kD / (16 * kPer);            // 64-byte chunks per row
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int sl = tid >> 2, sc = tid & 3;               // staging: rows 4sl .. 4sl + 3, bytes 16sc .. 16sc + 15
    const uint32_t rows = (uint32_t)(a.groups * a.rows_per_group), rpg = (uint32_t)a.rows_per_group;
    const uint32_t turns = (rows + kManyRows - 1) / kManyRows;
    const double* rw = sr + 8 * w;                       // wave w computes bits 8w .. 8w + 7
    const T* rp[kManyP];
    auto set_rows = [&](uint32_t uu) {
#pragma unroll
        for (int r = 0; r < kManyP; ++r) {
            const uint32_t rr = min(uu * kManyRows + kManyP * sl + r, rows - 1);
            rp[r] = static_cast<const T*>(a.x) + (int64_t)(rr / rpg) * a.x_group_stride + (int64_t)(rr % rpg) * kD +
                    sc * 4 * kPer;
        }
    };
    uint32_t u = blockIdx.x;                             // the grid is at most `turns` workgroups
    set_rows(u);
    // The first chunk is read with relaxed atomic loads: plain loads here would be merged with the
    // loop's prefetch into one load at the top of the loop, which would then wait at once.
    u32x4 pre[kManyP];
#pragma unroll
    for (int r = 0; r < kManyP; ++r) {
        const uint64_t* q = reinterpret_cast<const uint64_t*>(rp[r]);
        const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        pre[r] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
    }
    for (; u < turns; u += gridDim.x) {
        double acc[kManyP][8];
#pragma unroll
        for (int p = 0; p < kManyP; ++p)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[p][q] = 0.0;
        for (int k = 0; k < kChunks; ++k) {
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x4*>(&xs[(4 * sc + j) * kManyXs + kManyP * sl]) =
                    u32x4{pre[0][j], pre[1][j], pre[2][j], pre[3][j]};
            if (k + 1 < kChunks) {
#pragma unroll
                for (int r = 0; r < kManyP; ++r) pre[r] = ld16(rp[r] + (k + 1) * 16 * kPer);
            } else {                                     // the next turn's first chunk
                set_rows(min(u + gridDim.x, turns - 1));
#pragma unroll
                for (int r = 0; r < kManyP; ++r) pre[r] = ld16(rp[r]);
            }
            __syncthreads();
            for (int dw = 0; dw < 16; ++dw) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(&xs[dw * kManyXs + kManyP * lane]);
#pragma unroll
                for (int h = 0; h < kPer; ++h) {
                    const int e = (k * 16 + dw) * kPer + h;
                    double rv[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) rv[q] = rw[e * 32 + q];
#pragma unroll
                    for (int p = 0; p < kManyP; ++p) {
                        const float f = kPer == 1 ? __uint_as_float(v[p]) : h ? bf16_hi(v[p]) : bf16_lo(v[p]);
                        const double xv = (double)f;
#pragma unroll
                        for (int q = 0; q < 8; ++q) acc[p][q] = __fma_rn(xv, rv[q], acc[p][q]);
                    }
                }
            }
        }
        uint8_t* cb = reinterpret_cast<uint8_t*>(cs);   // byte w of a code holds bits 8w .. 8w + 7
#pragma unroll
        for (int p = 0; p < kManyP; ++p) {
            uint32_t v = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) v |= (acc[p][q] > 0.0 ? 1u : 0u) << q;
            cb[(kManyP * lane + p) * 4 + w] = (uint8_t)v;
        }
        __syncthreads();
        const uint32_t r = u * kManyRows + tid;
        if (r < rows) a.codes[(int64_t)(r / rpg) * a.codes_group_stride + (r % rpg)] = cs[tid];
    }
}

// Workgroups of the many-rows kernel one CU holds at once (cached; safe to
// call from several host threads).
template <typename T>
int many_slots_per_cu() {
    static std::atomic<int> slots{-1};
    int s = slots.load(std::memory_order_relaxed);
    if (s < 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&s, k_sig_encode_many<T>, 256, 0) != hipSuccess) s = 0;
        slots.store(s, std::memory_order_relaxed);
    }
    return s;
}

template <typename T>
hipError_t launch_many(const EncodeArgs& a, int64_t rows, hipStream_t st) {
    const int64_t turns = (rows + kManyRows - 1) / kManyRows;
    const int64_t slots = (int64_t)std::max(1, many_slots_per_cu<T>()) * std::max(1, device_cus());
    const dim3 grid((unsigned)std::min(turns, slots)), block(256);
    hipLaunchKernelGGL(k_sig_encode_many<T>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sig_encode(const EncodeArgs& a, hipStream_t st) {
    const int64_t rows = a.groups * a.rows_per_group;
    if (rows <= 0) return hipSuccess;
    if (rows >= kManyMinRows && rows <= INT32_MAX)
        return a.bf16 ? launch_many<uint16_t>(a, rows, st) : launch_many<float>(a, rows, st);
    const dim3 grid((unsigned)((rows + kRowsPerWg - 1) / kRowsPerWg)), block(64 * kEncWaves);
    if (a.bf16) hipLaunchKernelGGL(k_sig_encode<uint16_t>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(k_sig_encode<float>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace lcda
