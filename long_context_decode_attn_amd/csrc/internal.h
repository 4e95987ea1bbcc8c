// internal.h - host-side launch interfaces between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcda {

// Split attention over token ranges (or over a list of selected positions).
// Work unit = (KV batch item bkv, KV head h, row group rg); each unit owns
// `rows` query rows and reads one KV head.  Each unit's tokens are cut into
// `splits` ranges of `blocks_per_split` blocks; each (unit, split) writes one
// partial state per row into slot `split` of that row.
struct SplitArgs {
    const void* q;              // [B, Hq, d]
    const void* k;              // cache, element (bkv, h, j, c) at bkv*kv_batch_stride + (h*n + j)*d + c
    const void* v;
    int64_t kv_batch_stride;    // elements; 0 = one shared document
    int64_t n;                  // tokens per KV head in the cache layout
    const int32_t* n_b;         // per batch item valid length (<= n) or null
    const int32_t* idx;         // gather mode: [B, Hq, cap] positions; null = dense
    const int32_t* count;       // gather mode: [B, Hq]
    int64_t cap;
    int B, Hq, Hkv, G;
    int shared;                 // rows of a unit are (b, g) pairs over all b
    int rows;                   // query rows per (bkv, h)
    int row_groups;             // ceil(rows / rows_per_group)
    int splits;                 // slots per query row
    int blocks_per_split;       // split length in blocks of `block` tokens
    float2* ml;                 // partial states (see Partials)
    float* acc;
    // Arrival counters, one per unit (MFMA split, more than one split): the
    // last of a unit's `splits` workgroups to arrive combines the unit's rows
    // (see arrive_last).
    unsigned long long* ctr;
    float scale_log2;           // log2(e) / sqrt(d)
    // Fused cache + local step: tokens j >= n_c of row b come from k2 / v2
    // (local block, element (b, h, j - n_c, c) at b*kv2_batch_stride +
    // (h*n2 + j - n_c)*d + c); the row's token count is n_c + n2_b[b] (or + n2).
    const void* k2;             // null: no second segment
    const void* v2;
    int64_t n_c;
    int64_t n2;
    int64_t kv2_batch_stride;
    const int32_t* n2_b;
    // direct = 1 (one split): the split kernel finishes the rows itself,
    // merging the optional (a_in, alpha_in) pair, and writes out / alpha.
    int direct;
    float* out;                 // [B, Hq, d]
    float* alpha;               // [B, Hq] or null
    const float* a_in;          // [B, Hq, d] or null
    const float* alpha_in;      // [B, Hq] or null
};

// The scratch array of dense_decode_step_noalloc: at most this many query
// rows (B * Hq), and this many bytes in all (arrival counters included).
constexpr int kNoallocMaxRows = 8192;
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;

// Launch-shape knobs (process-wide; see lcda_set_tuning).
struct Tuning {
    int64_t dense_wgs = 256;       // target workgroups, MFMA split with 16/32-row tiles
    int64_t dense_wgs_nt4 = 256;   // target workgroups, MFMA split with 64-row tiles
    int64_t valu_wgs = 512;        // target workgroups, VALU dense split
    int64_t gather_wgs = 256;      // target workgroups, GATHER-ATT split (one per row in config 4: no combine)
    int64_t gather_waves = 8;      // GATHER-ATT wavefronts per workgroup (4, 8 or 16)
    int64_t direct_blocks = 16;    // at most this many blocks per unit: one split, no combine pass
    int64_t rows_wgs = 512;        // target workgroups, MFMA split with 64 rows per workgroup (shared document),
                                   // several 64-row groups per KV head (MFMA-bound: two workgroups per CU)
    int64_t rows_wgs_single = 256; // the same with one 64-row group per KV head (HBM-bound: one workgroup per
                                   // CU, half the partial states of two)
    int64_t rows_kernel = 1;       // bf16 with more than 16 rows per KV head: 1 = 64-row workgroups, 0 = 32/64-row wavefronts
    int64_t rows_variant = 8;      // 64-row workgroups: 0 = 4-slot ring, 2 per CU; 1 = 3 slots, 3 per CU;
                                   // 2 = 3 slots, 2 per CU; 3 = 2 slots, 3 per CU; 4-6 = blocks in registers
                                   // (4: cached loads, 2 per CU; 5: nontemporal; 6: cached, 1 per CU);
                                   // 7 = 5-slot ring, 2 per CU; 8 = two-tile wavefronts on
                                   // alternate blocks, 5-slot ring advanced by pairs, 2 per CU
    int64_t dense_variant = 0;     // MFMA split: 0 = nontemporal K/V loads, 1 = cached loads,
                                   // 2 = two blocks ahead, 3 = nontemporal with two waves per SIMD
    int64_t gather_variant = 0;    // GATHER-ATT rows: 0 = nontemporal loads, 1 = cached loads
    int64_t topk_subs = 0;         // TOPK: 4096-position sub-chunks per chunk (0: from topk_wgs)
    int64_t topk_wgs = 512;        // TOPK: workgroups a call aims at when topk_subs is 0
    int64_t topk_kernel = 1;       // TOPK: 1 = one launch with the distances kept in LDS and a histogram
                                   // exchange where the grid fits the device, 0 = chunked histogram +
                                   // compaction passes
    int64_t sparse_fused = 0;      // sparse_decode_step: 1 = SCORE + TOPK + GATHER-ATT in one launch where that
                                   // form applies, 0 = sig_score_topk then gather_attn
    int64_t topk_spin = 1 << 14;   // TOPK one-launch form: polls of the exchange wait before a workgroup counts
                                   // its partners' parts itself (0: at once; for tests of that path)
};
Tuning& tuning();

// Kernel variants for the split partial.
// kMfma16: split_mfma.hip, one wavefront per 16 / 32 query rows, the 4 wavefronts of a workgroup on
// different blocks.  kRows: split_rows.hip, 64 query rows per workgroup (one 16-row tile per
// wavefront), every block read once into LDS for all of them.  kValu: split_valu.hip.
enum SplitKernel { kMfma16 = 0, kValu = 1, kRows = 2 };

struct SplitPlan {
    int kernel;       // SplitKernel
    int nt;           // MFMA: 16-row tiles per wave (1, 2, 4); VALU: rows per group
    int waves;        // waves per workgroup
    int block;        // tokens per block (loop step of one wave)
    int rows_per_group;
    int row_groups;
    int splits;
    int blocks_per_split;
    int grid_x, grid_y, grid_z;
};

// Plan for a dense split over a cache of n tokens (gather: over cap positions).
SplitPlan plan_split(int dtype, bool gather, int B, int Hq, int Hkv, int64_t n_tokens,
                     bool shared);

hipError_t launch_split(const SplitPlan& p, const SplitArgs& a, int dtype, hipStream_t st);
hipError_t launch_split_mfma(const SplitPlan& p, const SplitArgs& a, hipStream_t st);
hipError_t launch_split_rows(const SplitPlan& p, const SplitArgs& a, hipStream_t st);
int split_rows_per_group();

// LSE combine of `slots` partial states per row (+ an optional virtual pair
// (a_in, alpha_in) per row) into out [rows, d] and alpha [rows].
struct CombineArgs {
    const float2* ml;
    const float* acc;
    int slots;
    int rows;
    const float* a_in;       // [rows, d] or null
    const float* alpha_in;   // [rows] natural log, or null
    float* out;
    float* alpha;            // may be null
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

// Records the formatted text that lcda_last_error returns and returns code.
int set_error(int code, const char* fmt, ...);

}  // namespace lcda
