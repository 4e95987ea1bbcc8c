/* lcda.h - decode-time attention of a few queries against a large cached K/V,
 * on AMD Instinct MI355X (gfx950).  C ABI of liblcda.so.
 *
 * Two paths:
 *   dense:  cached_attn_lse   - A(q) and alpha(q) against all cached tokens
 *           lse_merge_local   - exact merge of (A, alpha) with local tokens
 *   sparse: sig_encode        - T_map: random-projection codes of queries or new keys
 *           sig_score_topk    - HashAttention SCORE + TOPK over 32-bit codes
 *           sig_score_topk_q  - the same with the query codes encoded at its head
 *           sig_score_topk_w  - the same over codes of 2 to 16 words (64 to 512 bits)
 *           gather_attn       - attention renormalised over the selected rows
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array pointer is a DEVICE pointer (HIP device memory) unless the
 *   argument says otherwise.  The caller owns every buffer, including the
 *   workspace; the library never allocates, frees or synchronises.
 * - Every call only validates its arguments and enqueues kernels on `stream`
 *   (a hipStream_t; NULL = the default stream); it returns before the work
 *   completes.  A device fault surfaces at the caller's next synchronisation.
 * - Validation happens before any HIP call, so a non-OK status means nothing
 *   was enqueued (except LCDA_EHIP, reported by the launch itself).
 * - Buffers must not alias each other.  Array pointers must be 16-byte
 *   aligned.  Arrays are dense row-major with the shapes given.
 * - Head dimension d must be 128.  Query head hq reads KV head
 *   hq / (Hq / Hkv): query heads form contiguous groups of G = Hq / Hkv.
 * - Scores are s_j = q . k_j / sqrt(d); alpha is a natural logarithm.
 *   The scale is fixed by the method; there is no scale argument.
 * - Outputs and alphas are fp32.  q, K and V share one storage type: fp32 or
 *   bf16 (accumulation is fp32 either way).
 * - Empty sets (n = 0, count = 0, n_loc = 0 with alpha = -inf) give out = 0
 *   and alpha = -inf, never NaN.
 * - The status is an int: LCDA_OK or one of the LCDA_E* codes below; the text
 *   of the last failure on the calling thread is lcda_last_error().
 */
#ifndef LCDA_H
#define LCDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LCDA_F32 = 0, LCDA_BF16 = 1 } lcda_dtype;

enum {
    LCDA_OK = 0,
    LCDA_EINVAL = 1,       /* null required pointer, bad shape, misaligned pointer, cap too small */
    LCDA_EUNSUPPORTED = 2, /* d != 128, n > INT32_MAX, dtype not fp32/bf16 */
    LCDA_EWORKSPACE = 3,   /* ws_bytes smaller than the matching lcda_ws_bytes_* */
    LCDA_EHIP = 4          /* a HIP launch reported an error */
};

/* Dense attention with log-normalizer.
 *
 * Defines, for each batch item b and query head hq with KV head h:
 *   alpha(q) = log sum_j e^{s_j},   A(q) = sum_j e^{s_j} v_j / sum_j e^{s_j}
 * over all n cached tokens ("Nectar: Neural Estimation of Cached-Token
 * Attention via Regression", slide "Two functions separate retrieved content
 * from mass", Eq. (3.1)).  The sum is split over token ranges and the
 * partial results combined exactly through their log-normalizers (the
 * sequence-parallel decode the HashAttention slides compare against).
 *
 *   q      [B, Hq, d]                       dtype
 *   k, v   element (b, h, j, c) at b*kv_batch_stride + (h*n + j)*d + c   dtype
 *          kv_batch_stride (elements): 0 = one document shared by all B
 *          items, else >= Hkv*n*d
 *   out    [B, Hq, d] fp32    A(q)
 *   alpha  [B, Hq]    fp32    alpha(q)
 *   ws     workspace of at least lcda_ws_bytes_cached_attn_lse(...) bytes
 */
int cached_attn_lse(const void* q, const void* k, const void* v,
                    int B, int Hq, int Hkv, int d, int64_t n, int64_t kv_batch_stride,
                    int dtype, float* out, float* alpha,
                    void* ws, size_t ws_bytes, void* stream);

/* Exact merge with the visible local tokens.
 *
 * With Z_loc = sum_i e^{s_i} and N_loc = sum_i e^{s_i} v_i over the local
 * tokens i < n_loc[b]:
 *   out = (e^alpha A + N_loc) / (e^alpha + Z_loc),  alpha_out = log(e^alpha + Z_loc)
 * ("Nectar ...", slide "The score makes exact local attention composable",
 * Eq. (3.4)).  All n_loc[b] local tokens are visible (no mask).
 *
 *   q              [B, Hq, d]                 dtype
 *   a_in, alpha_in [B, Hq, d], [B, Hq]        fp32 (e.g. from cached_attn_lse;
 *                                             alpha_in = -inf: empty cached part)
 *   k_loc, v_loc   [B, Hkv, n_loc_max, d]     dtype (private per batch item)
 *   n_loc          [B] int32, 0 <= n_loc[b] <= n_loc_max; NULL = all n_loc_max
 *   out            [B, Hq, d] fp32
 *   alpha_out      [B, Hq] fp32, or NULL
 * out may not alias a_in.
 */
int lse_merge_local(const void* q, const float* a_in, const float* alpha_in,
                    const void* k_loc, const void* v_loc, const int32_t* n_loc,
                    int64_t n_loc_max, int B, int Hq, int Hkv, int d, int dtype,
                    float* out, float* alpha_out,
                    void* ws, size_t ws_bytes, void* stream);

/* HashAttention SCORE + TOPK.
 *
 * SCORE(k_i, q) = -popcount(h_i XOR h_q) over 32-bit codes ("HashAttention:
 * Semantic Sparsity for Faster Inference", slide "A 32-bit signature makes
 * scoring cheap", Eq. (2)).  TOPK picks the m positions of highest score
 * (smallest distance) over all n positions, ties to the lower position, and
 * unites them with the fixed windows [0, n_sink) and [n - n_recent, n)
 * (slides "Only selection is approximate; selected KV stay in full form" and
 * "Token-level sparsity still needs a careful kernel").  Each query head has
 * its own code and its own selected set I; the G query heads of a group read
 * the key codes of their KV head once.
 *
 *   key_sigs  [B, Hkv, n] uint32
 *   q_sigs    [B, Hq]     uint32
 *   idx       [B, Hq, cap] int32: I in ascending order, then -1 up to cap
 *   cap       >= min(n, m + n_sink + n_recent)
 *   count     [B, Hq] int32: |I|
 *   scores    [B, Hq, n] int8 = -distance, or NULL (not needed by the path)
 */
int sig_score_topk(const uint32_t* key_sigs, const uint32_t* q_sigs,
                   int B, int Hq, int Hkv, int64_t n, int64_t m, int64_t n_sink,
                   int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                   int8_t* scores, void* ws, size_t ws_bytes, void* stream);

/* sig_score_topk with the query codes encoded at its head (the T_map stage of
 * the query fused into the scan): q [B, Hq, 128] in q_dtype and R [128, bits]
 * fp32 as in sig_encode; q_sigs [B, Hq] uint32 receives the codes, and the
 * selection is the one sig_score_topk makes from them.  Everything else, the
 * workspace included, as in sig_score_topk. */
int sig_score_topk_q(const uint32_t* key_sigs, const void* q, int q_dtype, const float* R, int bits,
                     int B, int Hq, int Hkv, int64_t n, int64_t m, int64_t n_sink, int64_t n_recent,
                     int32_t* idx, int64_t cap, int32_t* count, int8_t* scores, uint32_t* q_sigs,
                     void* ws, size_t ws_bytes, void* stream);

/* SCORE + TOPK over codes of W 32-bit words (b = 32 W bits; W = 1, 2, 4, 8 or
 * 16): the distance popcount(h_i XOR h_q) of sig_score_topk summed over the
 * words, from 0 to b; the same selection, windows, order and padding.  These
 * are the code widths of HashAttention's scoring-cost sweep (64 to 512 bits;
 * slide with Table 6).  Three launches over chunks of each head: distances and
 * per-chunk histograms (a KV head's codes read once for up to 8 of its query
 * heads), the per-row threshold and chunk offsets, then ordered compaction.
 * W = 1 without scores (and at most 8 query heads per KV head) runs
 * sig_score_topk's kernel, which makes the same selection.
 *
 *   key_sigs  [B, Hkv, n, W] uint32 (word w of position i's code at i*W + w)
 *   q_sigs    [B, Hq, W]     uint32
 *   idx, cap, count          as in sig_score_topk
 *   scores    [B, Hq, n] int16 = -distance, or NULL
 *   ws        at least lcda_ws_bytes_sig_score_topk_w(B, Hq, n) bytes
 */
int sig_score_topk_w(const uint32_t* key_sigs, const uint32_t* q_sigs, int W, int B, int Hq, int Hkv, int64_t n,
                     int64_t m, int64_t n_sink, int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                     int16_t* scores, void* ws, size_t ws_bytes, void* stream);

/* T_map with a random projection: 32-bit codes of 128-value rows.
 *
 * Bit b of the code of row x is phi(x)_b = ReLU(sign(x . R[:, b])): 1 when
 * the projection is > 0, else 0 ("HashAttention ...", slide "A 32-bit
 * signature makes scoring cheap", Eq. (1), with F(x) = R^T x: the
 * random-projection selector of slide "Learning the codes matters more than
 * merely hashing"; the learned map needs trained weights).  Each projection is
 * a chain of fp64 fused multiply-adds over the 128 values in order, from 0:
 * codes are exact and reproducible, including the sign of a projection near
 * zero.  One call encodes queries (groups = 1, rows_per_group = B*Hq),
 * appends new keys' codes (groups = B*Hkv, one group per cached head), or
 * encodes a whole cache; from 16,384 rows a blocked kernel takes over (same
 * chains, same codes).
 *
 *   x      row (g, i), g < groups, i < rows_per_group, at
 *          x + g*x_group_stride + i*128 elements, dtype (fp32 or bf16);
 *          16-byte aligned, x_group_stride a multiple of 8
 *   R      [128, bits] fp32, 1 <= bits <= 32 (code bits at or past bits are 0)
 *   codes  row (g, i)'s code at codes[g*codes_group_stride + i] (uint32,
 *          4-byte aligned: e.g. key_sigs + n_old with codes_group_stride = n)
 * With groups > 1 the strides must not make rows overlap.  At most INT32_MAX
 * rows in all (LCDA_EUNSUPPORTED beyond).  No workspace.
 */
int sig_encode(const void* x, int dtype, int64_t groups, int64_t rows_per_group, int64_t x_group_stride,
               const float* R, int bits, uint32_t* codes, int64_t codes_group_stride, void* stream);

/* GATHER-ATT: attention over the selected rows only, renormalised over I:
 *   out = sum_{i in I} e^{s_i} v_i / sum_{j in I} e^{s_j},  alpha = log sum_{j in I} e^{s_j}
 * ("HashAttention ...", slide "Only selection is approximate; selected KV
 * stay in full form").  Rows are read straight from the cache by position
 * (page size 1, no gathered copy).
 *
 *   q, k, v, kv_batch_stride   as in cached_attn_lse (n cached tokens)
 *   idx    [B, Hq, cap] int32, the first count[b,hq] entries in [0, n)
 *   count  [B, Hq] int32, 0 <= count <= cap
 *   out    [B, Hq, d] fp32;  alpha [B, Hq] fp32 or NULL
 * Entries of idx outside [0, n) and counts outside [0, cap] are clamped into
 * range (no out-of-bounds access), and the results for such rows are undefined.
 */
int gather_attn(const void* q, const void* k, const void* v, int64_t kv_batch_stride,
                const int32_t* idx, const int32_t* count, int64_t cap,
                int B, int Hq, int Hkv, int d, int64_t n, int dtype,
                float* out, float* alpha, void* ws, size_t ws_bytes, void* stream);

/* Fused sparse decode step: sig_score_topk followed by gather_attn, in one
 * launch where possible.
 *
 * idx and count are sig_score_topk's (the selected set I of each query head,
 * ascending, -1 padded); out and alpha are gather_attn's over them
 * ("HashAttention ...", slides "Only selection is approximate; selected KV
 * stay in full form" and "Token-level sparsity still needs a careful
 * kernel": T = T_scan + T_TOPK + T_selected attention, here without a launch
 * or an index round trip between the terms).  The workgroups that select a
 * (batch item, KV head)'s positions then read those rows of the cache and
 * merge their partial softmax states exactly, as the split-KV pass does.
 * Results equal the two calls' up to floating-point summation order.  Falls
 * back to the two calls for shapes the one-launch form does not take (more
 * than 4 query heads per KV head, or a grid beyond one workgroup per CU).
 *
 *   key_sigs, q_sigs, m, n_sink, n_recent, idx, cap, count   as in sig_score_topk
 *   q, k, v, kv_batch_stride, n, dtype, out, alpha           as in gather_attn
 *   ws   at least lcda_ws_bytes_sparse_decode_step(...) bytes
 */
int sparse_decode_step(const uint32_t* key_sigs, const uint32_t* q_sigs, const void* q, const void* k,
                       const void* v, int64_t kv_batch_stride, int B, int Hq, int Hkv, int d, int64_t n,
                       int dtype, int64_t m, int64_t n_sink, int64_t n_recent, int32_t* idx, int64_t cap,
                       int32_t* count, float* out, float* alpha, void* ws, size_t ws_bytes, void* stream);

/* Fused dense decode step: cached_attn_lse followed by lse_merge_local, in
 * one pass where possible.
 *
 * out and alpha_out are the attention of q over the cached tokens and the
 * row's local tokens together, i.e. Eq. (3.4) of "Nectar ..." (slide "The
 * score makes exact local attention composable") applied to the (A, alpha)
 * of Eq. (3.1): the same quantities lse_merge_local returns after
 * cached_attn_lse, up to floating-point summation order.  Because the split
 * of the softmax sum is exact, the cached and local tokens are treated as one
 * token range: one split pass and one combine pass.  For a document shared by
 * B > 1 items (kv_batch_stride = 0) with more than 16 query rows per KV head,
 * the pass that reads each document block once for all rows also takes every
 * row's local tokens, as blocks that only that row's item sees.
 *
 *   q, k, v, kv_batch_stride, n          as in cached_attn_lse
 *   k_loc, v_loc, n_loc, n_loc_max       as in lse_merge_local
 *   out [B, Hq, d], alpha_out [B, Hq] (or NULL)   fp32
 *   a_doc [B, Hq, d], alpha_doc [B, Hq]  fp32, or both NULL: if given, they
 *        receive cached_attn_lse's (A, alpha), and the call runs as the two
 *        separate calls (the same happens for fp32 inputs, for a document
 *        shared by B > 1 items with at most 16 query rows per KV head or with
 *        n_loc_max = 0, and for n = 0)
 *   ws   at least lcda_ws_bytes_dense_decode_step(...) bytes
 */
int dense_decode_step(const void* q, const void* k, const void* v, int64_t kv_batch_stride, int64_t n,
                      const void* k_loc, const void* v_loc, const int32_t* n_loc, int64_t n_loc_max,
                      int B, int Hq, int Hkv, int d, int dtype,
                      float* out, float* alpha_out, float* a_doc, float* alpha_doc,
                      void* ws, size_t ws_bytes, void* stream);

/* dense_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The partial states and arrival counters
 * live in a static device array of the library, one per GPU, held until the
 * process ends: lcda_noalloc_scratch_bytes() bytes of workspace proper plus a
 * separate region for the counters.  The call allocates nothing.
 *
 *   arguments as in dense_decode_step, without a_doc, alpha_doc, ws, ws_bytes;
 *   stream must belong to the current device.
 * Errors: LCDA_EUNSUPPORTED when B*Hq exceeds 8192 query rows, or when the
 * workspace the call takes (its form, under the current lcda_set_tuning knobs)
 * exceeds lcda_noalloc_scratch_bytes() (16 MiB less the counters: a 61,440-token
 * shared document read by 16 items of 32 query heads needs 8.5 MB); the other
 * errors of dense_decode_step.  Every call on a GPU uses that GPU's one array:
 * calls that can overlap on one GPU (work on concurrent streams) race and
 * must not be issued. */
int dense_decode_step_noalloc(const void* q, const void* k, const void* v, int64_t kv_batch_stride, int64_t n,
                              const void* k_loc, const void* v_loc, const int32_t* n_loc, int64_t n_loc_max,
                              int B, int Hq, int Hkv, int d, int dtype,
                              float* out, float* alpha_out, void* stream);
size_t lcda_noalloc_scratch_bytes(void);

/* Workspace bytes each call needs for the given shapes (0 on invalid shapes). */
size_t lcda_ws_bytes_cached_attn_lse(int B, int Hq, int Hkv, int d, int64_t n,
                                     int64_t kv_batch_stride);
size_t lcda_ws_bytes_lse_merge_local(int B, int Hq, int Hkv, int d, int64_t n_loc_max);
size_t lcda_ws_bytes_sig_score_topk(int B, int Hq, int Hkv, int64_t n);
size_t lcda_ws_bytes_gather_attn(int B, int Hq, int Hkv, int d, int64_t cap);
size_t lcda_ws_bytes_sig_score_topk_w(int B, int Hq, int64_t n);
size_t lcda_ws_bytes_dense_decode_step(int B, int Hq, int Hkv, int d, int64_t n,
                                       int64_t kv_batch_stride, int64_t n_loc_max);
size_t lcda_ws_bytes_sparse_decode_step(int B, int Hq, int Hkv, int d, int64_t n, int64_t cap);

/* Text of the last non-OK status returned on the calling thread. */
const char* lcda_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* lcda_version(void);

/* Launch-shape knobs, for measurement and tuning (process-wide; set them
 * before enqueuing work, never concurrently with other calls).  They change
 * how work is split over workgroups, never what is computed.  Workspace sizes
 * (lcda_ws_bytes_*) do not depend on them: they cover every accepted setting,
 * so a knob changed after a workspace was sized (on any thread) never makes it
 * too small.  Keys (the *_wgs keys accept 1 .. 2048):
 *   "dense_wgs"      target workgroups of the MFMA split with 16/32-row tiles (256)
 *   "dense_wgs_nt4"  target workgroups of the MFMA split with 64-row tiles (256)
 *   "valu_wgs"       target workgroups of the fp32 dense split (512)
 *   "gather_wgs"     target workgroups of the GATHER-ATT split (256)
 *   "gather_waves"   GATHER-ATT wavefronts per workgroup: 4, 8 or 16 (8)
 *   "rows_wgs"       target workgroups of the MFMA split with 64 rows per workgroup,
 *                    used when more than 64 query rows read one KV head (512)
 *   "rows_wgs_single" the same when 17 to 64 query rows read one KV head (256)
 *   "rows_kernel"    more than 16 rows per KV head: 1 = 64-row workgroups sharing
 *                    each block through LDS, 0 = one wavefront per 32 / 64 rows (1)
 *   "rows_variant"   64-row workgroups: 0 = 4-slot LDS ring, 2 workgroups per CU;
 *                    1 = 3 slots, 3 per CU; 2 = 3 slots, 2 per CU; 3 = 2 slots, 3 per CU;
 *                    4-6 = every wavefront loads the block into registers (4: cached
 *                    loads, 2 workgroups per CU; 5: nontemporal; 6: cached, 1 per CU);
 *                    7 = 5-slot ring, 2 per CU; 8 = two 16-row tiles per wavefront, the
 *                    two wavefronts of each 32-row half on alternate blocks, 5-slot
 *                    ring, 2 per CU (8)
 *   "direct_blocks"  units with at most this many token blocks run as one split
 *                    that writes its rows directly, without a combine pass, when
 *                    the units alone reach the workgroup target (16)
 *   "dense_variant"  MFMA split K/V pipeline (16-row tiles): 0 = nontemporal
 *                    loads one block ahead, 1 = cached loads one block ahead,
 *                    2 = nontemporal two blocks ahead, 3 = as 0 with registers
 *                    capped so two workgroups share a CU; 4 = bf16 on the VALU
 *                    split instead of MFMA (dense_decode_step then takes the
 *                    two-call form), for comparison (0)
 *   "gather_variant" GATHER-ATT rows: 0 = nontemporal loads, 1 = cached loads (0)
 *   "topk_subs"      TOPK scans: 4096-position sub-chunks per workgroup (1..64;
 *                    more where a head would otherwise exceed 64 chunks); 0 picks
 *                    the count that gives about topk_wgs workgroups (0)
 *   "topk_wgs"       TOPK scans: workgroups a call aims at when topk_subs is 0 (512)
 *   "topk_kernel"    TOPK form: 1 = one launch that keeps the distances in LDS and
 *                    exchanges counts between the workgroups of a (b, KV head),
 *                    where its grid fits the device one workgroup per CU (at most 4
 *                    query heads per KV head and 64 steps of 4,096 positions);
 *                    0 = the chunked passes (1)
 *   "topk_spin"      one-launch TOPK: polls of a workgroup waiting for its partners
 *                    before it counts their share itself (16384, at most 2^20)
 *   "sparse_fused"   sparse_decode_step: 1 = SCORE + TOPK + GATHER-ATT in the one
 *                    TOPK launch where that form applies; 0 = sig_score_topk then
 *                    gather_attn (0)
 *   "wide_chunk"     sig_score_topk_w: positions per chunk, a multiple of 4096 up
 *                    to 32768 (raised where the workspace bound n / 2048 chunks
 *                    asks); 0 picks the length whose grid fills the device's
 *                    workgroup slots (0)
 * Returns LCDA_EINVAL for an unknown key or a negative (or, except
 * direct_blocks and wide_chunk, zero) value.  lcda_get_tuning returns -1 for an unknown key. */
int lcda_set_tuning(const char* key, int64_t value);
int64_t lcda_get_tuning(const char* key);

/* Streaming-read probe (not part of the method): reads `bytes` of device memory
 * at buf (16-byte aligned, bytes a multiple of 16) once, with `workgroups`
 * workgroups of 512 threads each keeping up to sixteen 16-byte nontemporal loads
 * in flight, and folds the words read into one value per thread; sink[0] (device,
 * 4 bytes) is written only by a thread whose value equals `never`.  Its rate is
 * the measured read ceiling that the kernels' HBM fractions are set against, next
 * to the published peak.  LCDA_EINVAL for a null or misaligned buf or sink, or
 * workgroups outside 1 .. 2^20; bytes = 0 does nothing. */
int lcda_stream_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, uint32_t never, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LCDA_H */
