/* oracle.c - plain, slow, obviously correct CPU oracle.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test-suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this.  It shares no code with
 * the GPU library.
 *
 * Sources followed (slide decks on the subject):
 *   [N]  "Nectar: Neural Estimation of Cached-Token Attention via Regression",
 *        slide "Two functions separate retrieved content from mass", Eq. (3.1);
 *        slide "The score makes exact local attention composable", Eq. (3.4).
 *   [HA] "HashAttention: Semantic Sparsity for Faster Inference",
 *        slide "Only selection is approximate; selected KV stay in full form"
 *        (exact o and sparse o-hat, the SCORE/TOPK/GATHER-ATT stages);
 *        slide "A 32-bit signature makes scoring cheap", Eq. (2);
 *        slide "Token-level sparsity still needs a careful kernel" (sink and
 *        recent windows, budget accounting);
 *        slide "Learning the codes matters more than merely hashing" (the
 *        random-projection LSH selector, whose codes sig_encode computes).
 *
 * Readings taken where the slides leave a step open are stated at each use.
 * Every sum is accumulated in double.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- input decoding ---------------------------------------------------- */

/* A bf16 value is the upper half of an IEEE binary32: shifting its 16 bits
 * left by 16 gives that binary32 exactly. */
static double bf16_bits_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element i of an array of the given storage type, as a double. */
static double elem(const void* base, int dtype, int64_t i) {
    if (dtype == ORC_F32) return (double)((const float*)base)[i];
    return bf16_bits_to_double(((const uint16_t*)base)[i]);
}

void orc_set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- softmax attention over an explicit list of tokens ------------------
 *
 * [N] Eq. (3.1): with s_j = q.k_j / sqrt(d),
 *     alpha = log sum_j e^{s_j},   A = sum_j e^{s_j} v_j / sum_j e^{s_j}.
 * [HA] o-hat is the same expression with j restricted to the selected set I.
 *
 * Numerator and denominator are both multiplied by e^{-M}, M = max_j s_j,
 * which leaves A unchanged and gives alpha = M + log(sum_j e^{s_j - M});
 * this only keeps e^{s_j} finite for large logits.
 *
 * tokens: the token positions to use (NULL = 0..cnt-1).  kb, vb point at the
 * first row of the KV head.  s: scratch of cnt doubles.  An empty list gives
 * A = 0 and alpha = -inf (the log of an empty sum). */
static void attend(const void* q, int dtype, int64_t q_off, const void* k, const void* v,
                   int64_t kv_off, const int32_t* tokens, int64_t cnt, int d,
                   double* s, double* out, double* alpha) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    if (cnt == 0) {
        *alpha = -INFINITY;
        return;
    }
    double M = -INFINITY;
    for (int64_t t = 0; t < cnt; ++t) {
        int64_t j = tokens ? tokens[t] : t;
        double dot = 0.0;
        for (int c = 0; c < d; ++c)
            dot += elem(q, dtype, q_off + c) * elem(k, dtype, kv_off + j * d + c);
        s[t] = dot * inv_sqrt_d;
        if (s[t] > M) M = s[t];
    }
    double Z = 0.0;
    for (int64_t t = 0; t < cnt; ++t) {
        int64_t j = tokens ? tokens[t] : t;
        double w = exp(s[t] - M);
        Z += w;
        for (int c = 0; c < d; ++c) out[c] += w * elem(v, dtype, kv_off + j * d + c);
    }
    for (int c = 0; c < d; ++c) out[c] /= Z;
    *alpha = M + log(Z);
}

/* ---- dense: A(q) and alpha(q) against all n cached tokens ([N] Eq. 3.1) - */

int orc_dense_attn(const void* q, const void* k, const void* v, int dtype,
                   int B, int Hq, int Hkv, int d, int64_t n, int64_t kv_batch_stride,
                   double* out, double* alpha) {
    if (!q || !out || !alpha || (n > 0 && (!k || !v))) return 1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || n < 0 || Hq % Hkv != 0) return 1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return 1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(2) schedule(dynamic)
        for (int b = 0; b < B; ++b)
            for (int hq = 0; hq < Hq; ++hq) {
                if (!s) continue;
                int h = hq / G;
                int64_t row = (int64_t)b * Hq + hq;
                attend(q, dtype, row * d, k, v, (int64_t)b * kv_batch_stride + (int64_t)h * n * d,
                       NULL, n, d, s, out + row * d, alpha + row);
            }
        free(s);
    }
    return bad ? 1 : 0;
}

/* ---- exact merge with the local tokens ([N] Eq. 3.4) --------------------
 *
 * Z_loc = sum_i e^{s_i}, N_loc = sum_i e^{s_i} v_i over the visible local
 * tokens i < n_loc[b] (all of them: the decode query is the newest position,
 * so no mask applies), and
 *     ATT_full = (e^alpha A + N_loc) / (e^alpha + Z_loc),
 *     alpha'   = log(e^alpha + Z_loc)   (log-normalizer of the union).
 * Numerator and denominator are multiplied by e^{-M'} with
 * M' = max(alpha, max_i s_i).  n_loc = 0 returns (A, alpha) unchanged; both
 * sides empty (alpha = -inf and n_loc = 0) returns 0 and -inf. */
int orc_merge_local(const void* q, int dtype, const double* a_in, const double* alpha_in,
                    const void* k_loc, const void* v_loc, const int32_t* n_loc,
                    int64_t n_loc_max, int B, int Hq, int Hkv, int d,
                    double* out, double* alpha_out) {
    if (!q || !a_in || !alpha_in || !out || !alpha_out) return 1;
    if (n_loc_max > 0 && (!k_loc || !v_loc)) return 1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || n_loc_max < 0 || Hq % Hkv != 0) return 1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return 1;
    if (n_loc)
        for (int b = 0; b < B; ++b)
            if (n_loc[b] < 0 || n_loc[b] > n_loc_max) return 1;
    const int G = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_loc_max > 0 ? n_loc_max : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(2) schedule(dynamic)
        for (int b = 0; b < B; ++b)
            for (int hq = 0; hq < Hq; ++hq) {
                if (!s) continue;
                int h = hq / G;
                int64_t row = (int64_t)b * Hq + hq;
                int64_t nl = n_loc ? n_loc[b] : n_loc_max;
                int64_t kv_off = ((int64_t)b * Hkv + h) * n_loc_max * d;
                const double* A = a_in + row * d;
                double alpha = alpha_in[row];
                double Mp = alpha;
                for (int64_t i = 0; i < nl; ++i) {
                    double dot = 0.0;
                    for (int c = 0; c < d; ++c)
                        dot += elem(q, dtype, row * d + c) * elem(k_loc, dtype, kv_off + i * d + c);
                    s[i] = dot * inv_sqrt_d;
                    if (s[i] > Mp) Mp = s[i];
                }
                double* o = out + row * d;
                if (Mp == -INFINITY) { /* nothing on either side */
                    for (int c = 0; c < d; ++c) o[c] = 0.0;
                    alpha_out[row] = -INFINITY;
                    continue;
                }
                double w_doc = exp(alpha - Mp); /* e^{alpha} / e^{M'} */
                double Z = w_doc;
                for (int c = 0; c < d; ++c) o[c] = w_doc * A[c];
                for (int64_t i = 0; i < nl; ++i) {
                    double w = exp(s[i] - Mp);
                    Z += w;
                    for (int c = 0; c < d; ++c) o[c] += w * elem(v_loc, dtype, kv_off + i * d + c);
                }
                for (int c = 0; c < d; ++c) o[c] /= Z;
                alpha_out[row] = Mp + log(Z);
            }
        free(s);
    }
    return bad ? 1 : 0;
}

/* ---- SCORE + TOPK ([HA] Eq. 2, the three stages, budget accounting) -----
 *
 * SCORE(k_i, q) = -popcount(h_i XOR h_q); the distance is counted with a
 * plain loop over the 32 bits.
 * TOPK: the m positions of smallest distance over all n positions.  Readings
 * (the slides do not fix these):
 *   - ties between equal distances go to the lower position;
 *   - the fixed windows (first n_sink, last n_recent positions) are united
 *     with the top m, so |I| <= m + n_sink + n_recent;
 *   - I is written in ascending position order, padded with -1 to cap.
 * Each query head has its own signature and its own I; it scans the key
 * signatures of its KV head hq / (Hq/Hkv). */

typedef struct {
    int dist;
    int64_t pos;
} dist_pos;

static int cmp_dist_pos(const void* a, const void* b) {
    const dist_pos* x = (const dist_pos*)a;
    const dist_pos* y = (const dist_pos*)b;
    if (x->dist != y->dist) return x->dist < y->dist ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

static int hamming32(uint32_t a, uint32_t b) {
    uint32_t x = a ^ b;
    int cnt = 0;
    for (int bit = 0; bit < 32; ++bit) cnt += (int)((x >> bit) & 1u);
    return cnt;
}

int orc_sig_topk(const uint32_t* key_sigs, const uint32_t* q_sigs,
                 int B, int Hq, int Hkv, int64_t n, int64_t m, int64_t n_sink,
                 int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                 int8_t* scores) {
    if (!q_sigs || !idx || !count || (n > 0 && !key_sigs)) return 1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 1;
    if (n < 0 || m < 0 || n_sink < 0 || n_recent < 0 || cap < 0 || n > 2147483647LL) return 1;
    /* the selected set can hold up to min(n, m + n_sink + n_recent) positions */
    if (cap < (m + n_sink + n_recent < n ? m + n_sink + n_recent : n)) return 1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        dist_pos* list = (dist_pos*)malloc(sizeof(dist_pos) * (size_t)(n > 0 ? n : 1));
        unsigned char* chosen = (unsigned char*)malloc((size_t)(n > 0 ? n : 1));
        if (!list || !chosen) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(2) schedule(dynamic)
        for (int b = 0; b < B; ++b)
            for (int hq = 0; hq < Hq; ++hq) {
                if (!list || !chosen) continue;
                int h = hq / G;
                int64_t row = (int64_t)b * Hq + hq;
                const uint32_t* ks = key_sigs + ((int64_t)b * Hkv + h) * n;
                uint32_t hqs = q_sigs[row];
                for (int64_t i = 0; i < n; ++i) {
                    list[i].dist = hamming32(ks[i], hqs);
                    list[i].pos = i;
                    if (scores) scores[row * n + i] = (int8_t)(-list[i].dist);
                    chosen[i] = 0;
                }
                qsort(list, (size_t)n, sizeof(dist_pos), cmp_dist_pos);
                int64_t take = m < n ? m : n;
                for (int64_t t = 0; t < take; ++t) chosen[list[t].pos] = 1;
                for (int64_t i = 0; i < n && i < n_sink; ++i) chosen[i] = 1;
                for (int64_t i = (n - n_recent > 0 ? n - n_recent : 0); i < n; ++i) chosen[i] = 1;
                int64_t c = 0;
                int overflow = 0;
                for (int64_t i = 0; i < n; ++i)
                    if (chosen[i]) {
                        if (c < cap) idx[row * cap + c] = (int32_t)i;
                        else overflow = 1;
                        ++c;
                    }
                for (int64_t t = c; t < cap; ++t) idx[row * cap + t] = -1;
                count[row] = (int32_t)(c < cap ? c : cap);
                if (overflow) {
#pragma omp atomic write
                    bad = 1;
                }
            }
        free(list);
        free(chosen);
    }
    return bad ? 1 : 0;
}

/* ---- GATHER-ATT ([HA] o-hat; renormalised over I) ----------------------- */

int orc_gather_attn(const void* q, const void* k, const void* v, int dtype,
                    int64_t kv_batch_stride, const int32_t* idx, const int32_t* count,
                    int64_t cap, int B, int Hq, int Hkv, int d, int64_t n,
                    double* out, double* alpha) {
    if (!q || !idx || !count || !out || !alpha || (n > 0 && (!k || !v))) return 1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || n < 0 || cap < 0 || Hq % Hkv != 0) return 1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return 1;
    for (int64_t r = 0; r < (int64_t)B * Hq; ++r) {
        if (count[r] < 0 || count[r] > cap) return 1;
        for (int64_t t = 0; t < count[r]; ++t)
            if (idx[r * cap + t] < 0 || idx[r * cap + t] >= n) return 1;
    }
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(2) schedule(dynamic)
        for (int b = 0; b < B; ++b)
            for (int hq = 0; hq < Hq; ++hq) {
                if (!s) continue;
                int h = hq / G;
                int64_t row = (int64_t)b * Hq + hq;
                attend(q, dtype, row * d, k, v, (int64_t)b * kv_batch_stride + (int64_t)h * n * d,
                       idx + row * cap, count[row], d, s, out + row * d, alpha + row);
            }
        free(s);
    }
    return bad ? 1 : 0;
}

/* ---- wider codes ---------------------------------------------------------- */

/* [HA] Eq. (2) with b = 32 W bits: the Hamming distance sums the bit
 * differences of all W words.  The selection is the one orc_sig_topk makes:
 * sort by (distance, position), take the first min(m, n), unite with the
 * windows, list ascending, pad with -1. */
int orc_sig_topk_w(const uint32_t* key_sigs, const uint32_t* q_sigs, int W,
                   int B, int Hq, int Hkv, int64_t n, int64_t m, int64_t n_sink,
                   int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                   int16_t* scores) {
    if (!q_sigs || !idx || !count || (n > 0 && !key_sigs)) return 1;
    if (W < 1 || W > 16 || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 1;
    if (n < 0 || m < 0 || n_sink < 0 || n_recent < 0 || cap < 0 || n > 2147483647LL) return 1;
    if (cap < (m + n_sink + n_recent < n ? m + n_sink + n_recent : n)) return 1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        dist_pos* list = (dist_pos*)malloc(sizeof(dist_pos) * (size_t)(n > 0 ? n : 1));
        unsigned char* chosen = (unsigned char*)malloc((size_t)(n > 0 ? n : 1));
        if (!list || !chosen) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for collapse(2) schedule(dynamic)
        for (int b = 0; b < B; ++b)
            for (int hq = 0; hq < Hq; ++hq) {
                if (!list || !chosen) continue;
                int h = hq / G;
                int64_t row = (int64_t)b * Hq + hq;
                const uint32_t* ks = key_sigs + ((int64_t)b * Hkv + h) * n * W;
                const uint32_t* qw = q_sigs + row * W;
                for (int64_t i = 0; i < n; ++i) {
                    int dist = 0;
                    for (int w = 0; w < W; ++w) dist += hamming32(ks[i * W + w], qw[w]);
                    list[i].dist = dist;
                    list[i].pos = i;
                    if (scores) scores[row * n + i] = (int16_t)(-dist);
                    chosen[i] = 0;
                }
                qsort(list, (size_t)n, sizeof(dist_pos), cmp_dist_pos);
                int64_t take = m < n ? m : n;
                for (int64_t t = 0; t < take; ++t) chosen[list[t].pos] = 1;
                for (int64_t i = 0; i < n && i < n_sink; ++i) chosen[i] = 1;
                for (int64_t i = (n - n_recent > 0 ? n - n_recent : 0); i < n; ++i) chosen[i] = 1;
                int64_t c = 0;
                int overflow = 0;
                for (int64_t i = 0; i < n; ++i)
                    if (chosen[i]) {
                        if (c < cap) idx[row * cap + c] = (int32_t)i;
                        else overflow = 1;
                        ++c;
                    }
                for (int64_t t = c; t < cap; ++t) idx[row * cap + t] = -1;
                count[row] = (int32_t)(c < cap ? c : cap);
                if (overflow) {
#pragma omp atomic write
                    bad = 1;
                }
            }
        free(list);
        free(chosen);
    }
    return bad ? 1 : 0;
}

/* ---- T_map: random-projection signatures ---------------------------------- */

/* phi(x) = ReLU(sign(F(x))) with F(x) = R^T x, [HA] Eq. (1); component b is
 * bit b of the code.  sign(0) = 0, so a zero projection gives bit 0. */
int orc_sig_encode(const void* x, int dtype, int64_t rows, int d, const float* R, int bits, uint32_t* codes) {
    if (rows < 0 || d <= 0 || bits <= 0 || bits > 32 || (rows > 0 && (!x || !R || !codes))) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        uint32_t c = 0;
        for (int b = 0; b < bits; ++b) {
            double z = 0.0;
            for (int e = 0; e < d; ++e) z = fma(elem(x, dtype, i * d + e), (double)R[(int64_t)e * bits + b], z);
            if (z > 0.0) c |= 1u << b;
        }
        codes[i] = c;
    }
    return 0;
}
