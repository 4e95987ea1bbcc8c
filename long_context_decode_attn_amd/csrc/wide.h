// wide.h - host-side launch interface of SCORE + TOPK over codes of W words
// (sig_topk_wide.hip).
#pragma once

#include "internal.h"

namespace lcda {

// Signature top-k over codes of W words (histogram, select and compaction passes
// over chunks of L positions; workgroups of the first and last pass take a KV
// head's group of HG query heads).
struct WideArgs {
    const uint32_t* key_sigs;   // [B, Hkv, n, W]
    const uint32_t* q_sigs;     // [B, Hq, W]
    int W, B, Hq, Hkv, G;
    int HG, ng;                 // query heads per group (wide_group(G)) and groups per KV head
    int64_t n, m, n_sink, n_recent, cap;
    int64_t L, nc;              // chunk length (a multiple of wide_granule(W), <= kWideMaxL) and chunks per head
    bool vec;                   // 16-byte loads of the codes are aligned (base aligned, n * W % 4 == 0)
    int32_t* idx;               // [B, Hq, cap]
    int32_t* count;             // [B, Hq]
    int16_t* scores;            // [B, Hq, n] or null
    // workspace
    uint8_t* dist;              // [B, Hkv, ng][dstride] bytes: min(distance, 255) of a group's HG heads,
                                // position-major ([n][HG]), for W >= 2
    int64_t dstride;            // bytes per (b, KV head, group): a multiple of 16, >= round_up(n, 16) * HG
    uint16_t* hist;             // [3][B * Hq][nc][32 W + 1 padded to 8]: all positions, sink part, recent part
    uint32_t* rec;              // [B * Hq][nc][2]: ties at t before the chunk, positions selected before it
    int32_t* rowrec;            // [B * Hq][2]: t, quota
};
constexpr int64_t kWideMaxL = 32768;   // positions per chunk at most (16-bit histogram counts)
constexpr int64_t kWideMinL = 2048;    // and at least, where n allows (bounds the workspace)
int wide_group(int G);
int wide_slots_per_cu(int W, int HG);  // workgroups of the chunk passes one CU holds at once
int wide_granule(int W);               // chunk lengths are multiples: whole histogram-loop turns and compaction tiles

hipError_t launch_topk_wide(const WideArgs& a, hipStream_t st);

}  // namespace lcda
