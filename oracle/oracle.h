/* oracle.h - plain CPU oracle for decode attention against a large cached K/V.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark may call anything declared here.
 * It shares no source with the GPU library: no header, helper, table or
 * constant is common to both.
 *
 * Every floating-point quantity is accumulated in double.  Inputs are read as
 * given: fp32 is widened, bf16 bit patterns are expanded exactly.
 *
 * Layouts (row-major, contiguous):
 *   q      [B, Hq, d]
 *   k, v   element (b, h, j, c) at  b*kv_batch_stride + (h*n + j)*d + c
 *          (kv_batch_stride == 0: one document shared by every batch item)
 *   query head hq reads KV head hq / (Hq/Hkv)   (contiguous GQA groups)
 *
 * Status: 0 = OK, 1 = invalid argument.
 */
#ifndef LCDA_ORACLE_H
#define LCDA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* Dense attention of each query against all n cached tokens:
 * out = A(q) and alpha = alpha(q) of Nectar's Eq. (3.1). */
int orc_dense_attn(const void* q, const void* k, const void* v, int dtype,
                   int B, int Hq, int Hkv, int d, int64_t n, int64_t kv_batch_stride,
                   double* out, double* alpha);

/* Exact merge of (A, alpha) with the visible local tokens, Nectar's Eq. (3.4).
 * k_loc, v_loc: [B, Hkv, n_loc_max, d]; n_loc: [B] or NULL (all n_loc_max). */
int orc_merge_local(const void* q, int dtype, const double* a_in, const double* alpha_in,
                    const void* k_loc, const void* v_loc, const int32_t* n_loc,
                    int64_t n_loc_max, int B, int Hq, int Hkv, int d,
                    double* out, double* alpha_out);

/* HashAttention SCORE + TOPK: distances popcount(h_i XOR h_q), the m smallest
 * (ties to the lower index) united with the sink [0,s) and recent [n-r,n)
 * windows, written ascending and padded with -1 up to cap.
 * key_sigs [B, Hkv, n], q_sigs [B, Hq]; idx [B, Hq, cap]; count [B, Hq];
 * scores [B, Hq, n] (= -distance) or NULL. */
int orc_sig_topk(const uint32_t* key_sigs, const uint32_t* q_sigs,
                 int B, int Hq, int Hkv, int64_t n, int64_t m, int64_t n_sink,
                 int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                 int8_t* scores);

/* GATHER-ATT: Eq. (3.1) restricted to the selected set I = idx[b,hq,0:count). */
int orc_gather_attn(const void* q, const void* k, const void* v, int dtype,
                    int64_t kv_batch_stride, const int32_t* idx, const int32_t* count,
                    int64_t cap, int B, int Hq, int Hkv, int d, int64_t n,
                    double* out, double* alpha);

/* SCORE + TOPK over codes of W 32-bit words (b = 32 W bits, 1 <= W <= 16):
 * the distance is the popcount of the XOR over all W words, so it runs from 0
 * to b; selection, windows, order and padding as in orc_sig_topk.  The wider
 * codes are the ones HashAttention's code-width sweep scores (slide "Table 6:
 * scoring cost", 64 to 512 bits).  key_sigs [B, Hkv, n, W], q_sigs [B, Hq, W];
 * scores [B, Hq, n] int16 (= -distance) or NULL. */
int orc_sig_topk_w(const uint32_t* key_sigs, const uint32_t* q_sigs, int W,
                   int B, int Hq, int Hkv, int64_t n, int64_t m, int64_t n_sink,
                   int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                   int16_t* scores);

/* T_map with a random projection (the LSH selector HashAttention compares
 * against): code bit b of row i is phi(x_i)_b = ReLU(sign(z_b)), i.e. 1 when
 * z_b = sum_e x[i][e] * R[e][b] > 0 and 0 otherwise ("A 32-bit signature makes
 * scoring cheap", Eq. (1)).  x: [rows, d] in dtype, R: [d, bits] float32 with
 * bits <= 32, codes: [rows].  z_b is accumulated as a chain of fused
 * multiply-adds in double, e = 0 .. d-1 in order, from 0: every product of a
 * bf16 or float32 value with a float32 value is exact in double, and the chain
 * fixes the rounding of the sum, so the sign of a near-zero z_b is
 * reproducible. */
int orc_sig_encode(const void* x, int dtype, int64_t rows, int d, const float* R, int bits, uint32_t* codes);

/* OpenMP thread count used by the calls above (<= 0: leave the default). */
void orc_set_threads(int nthreads);
int orc_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif
