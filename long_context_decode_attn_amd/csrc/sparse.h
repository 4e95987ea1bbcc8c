// sparse.h - host-side launch interfaces of the sparse path's kernels: the
// signature encoder (T_map), SCORE + TOPK over one-word codes and the
// one-launch SCORE + TOPK (+ GATHER-ATT) form.
#pragma once

#include "internal.h"

namespace lcda {

// Random-projection codes (T_map).
struct EncodeArgs {
    const void* x;             // row (g, i) at x + g * x_group_stride + i * 128 elements
    bool bf16;                 // x is bf16 (else fp32)
    int64_t groups, rows_per_group, x_group_stride;
    const float* R;            // [128, bits]
    int bits;                  // 1 .. 32
    uint32_t* codes;           // row (g, i) at codes[g * codes_group_stride + i]
    int64_t codes_group_stride;
};
hipError_t launch_sig_encode(const EncodeArgs& a, hipStream_t st);

// Signature top-k.
struct TopkArgs {
    const uint32_t* key_sigs;   // [B, Hkv, n]
    const uint32_t* q_sigs;     // [B, Hq]
    int B, Hq, Hkv, G;
    int64_t n, m, n_sink, n_recent, cap;
    int32_t* idx;               // [B, Hq, cap]
    int32_t* count;             // [B, Hq]
    int8_t* scores;             // [B, Hq, n] or null
    uint32_t* hist;             // ws: [B, Hq, chunks + 2, topk_hist_row()] distance histograms of each
                                // chunk, then of the sink part and the recent part of the chunks a
                                // window edge cuts
    const void* q;              // [B, Hq, 128] or null: the histogram pass encodes the query codes itself
    bool q_bf16;                // (with R [128, bits]) and writes them to q_codes, which the
    const float* R;             // compaction then reads
    int bits;
    uint32_t* q_codes;          // [B, Hq]: where the encoded query codes go
    int chunks;                 // ceil(n / chunk_len) <= 64
    int64_t chunk_len;
    // One launch with two exchanges (sig_topk_unit.hip): each (b, KV head)
    // unit's steps of 4,096 positions dealt round robin to `parts` workgroups,
    // part_len / 4096 steps each.
    int parts;
    int part_len;
    unsigned long long* bar;    // ws: [B * Hkv] arrival counters of the histogram exchange
    uint32_t* epoch;            // ws: [B * Hkv] its release epochs
    uint32_t* phist;            // ws: [B * Hkv][parts][4][topk_unit_row_words()] published histograms
    unsigned long long* rbar;   // ws: [B * Hkv] arrival counters of the step-record exchange
    uint32_t* repoch;           // ws: [B * Hkv] its release epochs
    uint32_t* srec;             // ws: [B * Hkv][topk_unit_rec_words()] published step records
    int spin_max;               // polls of an exchange wait
    // GATHER-ATT of the selected rows in the same launch (sparse_decode_step;
    // one-launch form only): gk == null means TOPK alone.
    const void* gq;             // [B, Hq, 128]
    const void* gk;             // cache as in SplitArgs::k
    const void* gv;
    int64_t kv_batch_stride;    // elements; 0 = one shared document
    float* out;                 // [B, Hq, 128]
    float* alpha;               // [B, Hq] or null
    float2* pml;                // ws: [B * Hq][parts] partial (m, l) of each part
    float* pacc;                // ws: [B * Hq][parts][128] partial sums of each part
    unsigned long long* bar2;   // ws: [B * Hkv] arrival counters of the merge
    float scale_log2;           // log2(e) / sqrt(d)
};
int topk_chunk_len(int64_t n, int units);   // units: B * Hkv
// One launch per call with exchanges between workgroups (sig_topk_unit.hip):
// positions per part (4096 x steps) of a (b, KV head) unit, 0 when that form
// does not apply (G > 4, more than 64 steps of 4,096 positions, or the grid of
// units x parts exceeds `cus` workgroups, one per CU).
int topk_unit_part(int64_t n, int units, int G, int cus);
int topk_unit_row_words();
int topk_unit_rec_words();
// dtype: the rows' type when a.gk is set (LCDA_F32 or LCDA_BF16).
hipError_t launch_topk_unit(const TopkArgs& a, int dtype, hipStream_t st);
int topk_hist_row();
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

}  // namespace lcda
