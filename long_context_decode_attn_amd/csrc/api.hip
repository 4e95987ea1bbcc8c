// api.hip - the C ABI of liblcda: argument validation, workspace layout, launch
// planning and kernel launches on the caller's stream.  Validation finishes
// before any HIP call.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "../../include/lcda.h"
#include "common.h"
#include "device.h"
#include "internal.h"
#include "sparse.h"
#include "wide.h"

namespace lcda {

hipError_t launch_split_valu(const SplitPlan& p, const SplitArgs& a, int dtype, bool gather, hipStream_t st);
int valu_step_tokens();

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

}  // namespace

// The same, for the library's other source files.
int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// lcda_set_tuning "wide_chunk": positions per chunk of sig_score_topk_w (0:
// from the device's workgroup slots).  Kept here, not in Tuning: the split
// kernels' sources do not change with the wide path's knobs.
int64_t g_wide_chunk = 0;
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t elem_bytes(int dtype) { return dtype == LCDA_F32 ? 4 : 2; }

// Shape checks shared by the attention calls.
int check_heads(const char* fn, int B, int Hq, int Hkv, int d) {
    if (d != kD) return fail(LCDA_EUNSUPPORTED, "%s: d = %d, only d = 128 is supported", fn, d);
    if (B < 0) return fail(LCDA_EINVAL, "%s: B = %d < 0", fn, B);
    if (Hq <= 0 || Hkv <= 0) return fail(LCDA_EINVAL, "%s: Hq = %d, Hkv = %d must be positive", fn, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(LCDA_EINVAL, "%s: Hq = %d is not a multiple of Hkv = %d", fn, Hq, Hkv);
    return LCDA_OK;
}

int check_dtype(const char* fn, int dtype) {
    if (dtype != LCDA_F32 && dtype != LCDA_BF16)
        return fail(LCDA_EUNSUPPORTED, "%s: dtype %d is neither LCDA_F32 nor LCDA_BF16", fn, dtype);
    return LCDA_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, bool required) {
    if (!p) return required ? fail(LCDA_EINVAL, "%s: %s is NULL", fn, name) : LCDA_OK;
    if (!aligned16(p)) return fail(LCDA_EINVAL, "%s: %s is not 16-byte aligned", fn, name);
    return LCDA_OK;
}

int check_n(const char* fn, const char* name, int64_t n) {
    if (n < 0) return fail(LCDA_EINVAL, "%s: %s = %lld < 0", fn, name, (long long)n);
    if (n > INT32_MAX) return fail(LCDA_EUNSUPPORTED, "%s: %s = %lld exceeds INT32_MAX", fn, name, (long long)n);
    return LCDA_OK;
}

int check_kv_stride(const char* fn, int64_t stride, int Hkv, int64_t n, int dtype) {
    if (stride < 0) return fail(LCDA_EINVAL, "%s: kv_batch_stride < 0", fn);
    if (stride != 0 && stride < (int64_t)Hkv * n * kD)
        return fail(LCDA_EINVAL, "%s: kv_batch_stride %lld < Hkv*n*d = %lld", fn, (long long)stride,
                    (long long)((int64_t)Hkv * n * kD));
    if ((stride * (int64_t)elem_bytes(dtype)) % 16 != 0)
        return fail(LCDA_EINVAL, "%s: kv_batch_stride*element size is not a multiple of 16 bytes", fn);
    return LCDA_OK;
}

// Workspace of a split pass: one arrival counter per work unit (at most one
// unit per query row), then the partial states of every (row, split) slot.
struct PartialLayout {
    size_t ctr_off, ml_off, acc_off, bytes;
};

PartialLayout partial_layout(int B, int Hq, int splits, bool own_ctr = true) {
    PartialLayout l;
    const size_t slots = (size_t)B * Hq * splits;
    l.ctr_off = 0;
    l.ml_off = own_ctr ? round_up((size_t)B * Hq * sizeof(unsigned long long)) : 0;
    l.acc_off = l.ml_off + round_up(slots * sizeof(float2));
    l.bytes = l.acc_off + round_up(slots * kD * sizeof(float));
    return l;
}

// Where a call's scratch memory lives: the workspace (bytes at ws), and the
// arrival counters either at the start of it (ctr == null) or in a region of
// their own that holds nothing else.
struct Scratch {
    void* ws;
    size_t bytes;
    unsigned long long* ctr;
};

unsigned long long* counters_at(const Scratch& s, const PartialLayout& l) {
    return s.ctr ? s.ctr : reinterpret_cast<unsigned long long*>(static_cast<char*>(s.ws) + l.ctr_off);
}

#define RETURN_IF(x)          \
    do {                      \
        int _s = (x);         \
        if (_s != LCDA_OK) return _s; \
    } while (0)

int hip_status(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(LCDA_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return LCDA_OK;
}

// Launch the split pass, then the combine pass unless the plan has a single
// split (the split kernel then writes the final rows itself) or the split
// kernel combines each unit itself (kMfma16: the last workgroup of a unit to
// finish merges its rows).  kRows units are too large for that, and for the
// short gather units of kValu the arrival at the end of every workgroup costs
// more than the separate pass.
int finish(const char* fn, const SplitPlan& p, SplitArgs& a, int dtype, int rows, float* out, float* alpha,
           const float* a_in, const float* alpha_in, hipStream_t st) {
    a.direct = p.splits == 1 ? 1 : 0;
    a.out = out;
    a.alpha = alpha;
    a.a_in = a_in;
    a.alpha_in = alpha_in;
    RETURN_IF(hip_status(fn, launch_split(p, a, dtype, st)));
    if (a.direct || p.kernel == kMfma16) return LCDA_OK;
    CombineArgs c{};
    c.ml = a.ml;
    c.acc = a.acc;
    c.slots = p.splits;
    c.rows = rows;
    c.a_in = a_in;
    c.alpha_in = alpha_in;
    c.out = out;
    c.alpha = alpha;
    return hip_status(fn, launch_combine(c, st));
}

// Workspace of sig_score_topk, sized for either TOPK form whatever the launch
// knobs: the chunked form's distance histograms of every chunk (at most
// kTopkMaxChunks) and of the two window parts, or the one-launch form's arrival
// counters, epochs, published part histograms (at most 64 parts per unit) and
// step records.  Both forms start at offset 0; a call uses one of them.
constexpr int kTopkMaxChunks = 64;

struct TopkLayout {
    size_t bar_off, epoch_off, phist_off, rbar_off, repoch_off, srec_off;
    size_t bytes;
};

// The chunked passes' histograms, or the one-launch form's counters, epochs,
// published histograms and step records (whichever is larger: the two forms
// share the space, and which one runs does not change the size).
TopkLayout topk_layout(int B, int Hq, int Hkv, int64_t n) {
    TopkLayout l;
    const size_t rows = (size_t)B * Hq, units = (size_t)B * Hkv;
    const size_t chunked = round_up(rows * (kTopkMaxChunks + 2) * topk_hist_row() * sizeof(uint32_t));
    const size_t max_parts = (size_t)std::min<int64_t>(64, std::max<int64_t>(1, (n + 4095) / 4096));
    l.bar_off = 0;
    l.epoch_off = round_up(units * sizeof(unsigned long long));
    l.phist_off = l.epoch_off + round_up(units * sizeof(uint32_t));
    l.rbar_off = l.phist_off + round_up(units * max_parts * 4 * topk_unit_row_words() * sizeof(uint32_t));
    l.repoch_off = l.rbar_off + round_up(units * sizeof(unsigned long long));
    l.srec_off = l.repoch_off + round_up(units * sizeof(uint32_t));
    const size_t unit = l.srec_off + round_up(units * topk_unit_rec_words() * sizeof(uint32_t));
    l.bytes = std::max(chunked, unit);
    return l;
}

// The one-launch form's exchange buffers in workspace w.
void set_unit_ws(TopkArgs& a, char* w, const TopkLayout& l) {
    a.bar = reinterpret_cast<unsigned long long*>(w + l.bar_off);
    a.epoch = reinterpret_cast<uint32_t*>(w + l.epoch_off);
    a.phist = reinterpret_cast<uint32_t*>(w + l.phist_off);
    a.rbar = reinterpret_cast<unsigned long long*>(w + l.rbar_off);
    a.repoch = reinterpret_cast<uint32_t*>(w + l.repoch_off);
    a.srec = reinterpret_cast<uint32_t*>(w + l.srec_off);
}

}  // namespace

Tuning& tuning() {
    static Tuning t;
    return t;
}

// Token range of a fused step: the cache tokens, padded to whole 32-token
// blocks, then the local tokens (so no block spans both).
int64_t fused_tokens(int64_t n, int64_t n_loc_max) { return (n + 31) / 32 * 32 + n_loc_max; }

namespace {

// The split plan under the knobs in t (plan_split uses the current ones).
SplitPlan plan_split_t(const Tuning& t, int dtype, bool gather, int B, int Hq, int Hkv, int64_t n_tokens,
                       bool shared);

}  // namespace

SplitPlan plan_split(int dtype, bool gather, int B, int Hq, int Hkv, int64_t n_tokens, bool shared) {
    return plan_split_t(tuning(), dtype, gather, B, Hq, Hkv, n_tokens, shared);
}

namespace {

SplitPlan plan_split_t(const Tuning& t, int dtype, bool gather, int B, int Hq, int Hkv, int64_t n_tokens,
                       bool shared) {
    SplitPlan p{};
    const int G = Hq / Hkv;
    const int rows = shared ? B * G : G;
    const int bkv = shared ? 1 : B;
    int units, target;
    p.waves = 4;
    if (gather) {
        p.kernel = kValu;
        p.nt = 1;
        p.rows_per_group = 1;
        p.row_groups = 1;
        p.block = valu_step_tokens();
        units = B * Hq;
        p.waves = (int)t.gather_waves;
        target = (int)t.gather_wgs;
        p.grid_y = Hq;
        p.grid_z = B;
    } else if (dtype == LCDA_BF16 && rows > 16 && t.rows_kernel) {
        // Many rows per KV head (a shared document): 64 rows per workgroup, every block read once.
        p.kernel = kRows;
        p.nt = 1;
        p.waves = 1;   // the wavefronts split rows, not tokens
        p.rows_per_group = split_rows_per_group();
        p.row_groups = (int)ceil_div(rows, p.rows_per_group);
        p.block = 32;
        units = bkv * Hkv * p.row_groups;
        target = (int)(p.row_groups == 1 ? t.rows_wgs_single : t.rows_wgs);
        p.grid_y = Hkv;
        p.grid_z = bkv * p.row_groups;
    } else if (dtype == LCDA_BF16 && t.dense_variant != 4) {
        p.kernel = kMfma16;
        p.nt = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
        p.rows_per_group = 16 * p.nt;
        p.row_groups = (int)ceil_div(rows, p.rows_per_group);
        p.block = 32;
        units = bkv * Hkv * p.row_groups;
        target = (int)(p.nt == 4 ? t.dense_wgs_nt4 : t.dense_wgs);
        p.grid_y = Hkv;
        p.grid_z = bkv * p.row_groups;
    } else {
        p.kernel = kValu;
        p.rows_per_group = rows >= 3 ? 4 : (rows > 0 ? rows : 1);
        p.nt = p.rows_per_group;
        p.row_groups = (int)ceil_div(rows, p.rows_per_group);
        p.block = valu_step_tokens();
        units = bkv * Hkv * p.row_groups;
        target = (int)t.valu_wgs;
        p.grid_y = Hkv;
        p.grid_z = bkv * p.row_groups;
    }
    const int64_t nblocks = n_tokens > 0 ? ceil_div(n_tokens, p.block) : 0;
    const int64_t max_splits = nblocks > 0 ? ceil_div(nblocks, p.waves) : 1;
    int64_t splits = ceil_div(target, units > 0 ? units : 1);
    // Short ranges run as one split finished in place, unless there are too few
    // units to fill the chip that way.
    if (nblocks <= t.direct_blocks && units >= target) splits = 1;
    splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
    splits = std::min<int64_t>(splits, kCtrMaxTarget);   // an arrival counter counts at most this many
    const int64_t bps = nblocks > 0 ? ceil_div(nblocks, splits) : 1;
    splits = nblocks > 0 ? ceil_div(nblocks, bps) : 1;
    p.splits = (int)splits;
    p.blocks_per_split = (int)bps;
    p.grid_x = p.splits;
    return p;
}

// Target workgroups accepted by lcda_set_tuning (its *_wgs keys).
constexpr int64_t kMaxTargetWgs = 2048;

// The largest split count any accepted knob setting gives a shape: the
// workspace sizes (lcda_ws_bytes_*) follow it, so that lcda_set_tuning never
// makes a workspace sized earlier too small.  More target workgroups, fewer
// GATHER-ATT wavefronts and no direct runs only ever add splits; rows_kernel
// and dense_variant 4 pick between kernels, so each choice is tried.
int max_plan_splits(int dtype, bool gather, int B, int Hq, int Hkv, int64_t n_tokens, bool shared) {
    int s = 1;
    for (int rk = 0; rk <= 1; ++rk) {
        for (int dv : {0, 4}) {   // dense_variant 4 puts bf16 on the VALU split
            Tuning t = tuning();
            t.dense_wgs = t.dense_wgs_nt4 = t.valu_wgs = t.gather_wgs = t.rows_wgs = t.rows_wgs_single =
                kMaxTargetWgs;
            t.gather_waves = 4;
            t.direct_blocks = 0;
            t.rows_kernel = rk;
            t.dense_variant = dv;
            s = std::max(s, plan_split_t(t, dtype, gather, B, Hq, Hkv, n_tokens, shared).splits);
        }
    }
    return s;
}

// Workspace of one split pass: under the current knobs (any = false) or under
// any accepted ones (any = true).
size_t split_ws(int dtype, bool gather, int B, int Hq, int Hkv, int64_t n_tokens, bool shared, bool any) {
    const int s = any ? max_plan_splits(dtype, gather, B, Hq, Hkv, n_tokens, shared)
                      : plan_split(dtype, gather, B, Hq, Hkv, n_tokens, shared).splits;
    return partial_layout(B, Hq, s).bytes;
}

}  // namespace

// Workspace of dense_decode_step in the form a call with these arguments takes
// (the 64-row shared-document pass, the two calls, or the fused split), under
// the current knobs (any = false) or any accepted ones (any = true, where the
// form a knob could switch to is covered as well).
size_t dense_step_ws(int dtype, int B, int Hq, int Hkv, int64_t n, int64_t kv_batch_stride, int64_t n_loc_max,
                     bool a_doc, bool any) {
    const bool shared = kv_batch_stride == 0 && B > 1;
    size_t need = 0;
    if (shared && dtype == LCDA_BF16 && !a_doc && n > 0 && n_loc_max > 0) {
        const SplitPlan p = plan_split(dtype, false, B, Hq, Hkv, n, true);
        const size_t rows = split_ws(dtype, false, B, Hq, Hkv, n, true, any);
        if (p.kernel == kRows && !any) return rows;
        need = rows;
    }
    if (dtype != LCDA_BF16 || shared || a_doc || n == 0 || any || tuning().dense_variant == 4) {
        // the two calls: each one's workspace, then the doc-only (A, alpha)
        need = std::max(need, split_ws(dtype, false, B, Hq, Hkv, n, kv_batch_stride == 0, any) +
                                  split_ws(dtype, false, B, Hq, Hkv, n_loc_max, false, any) +
                                  round_up((size_t)B * Hq * (kD + 1) * sizeof(float)));
        if (!any) return need;
    }
    return std::max(need, split_ws(dtype, false, B, Hq, Hkv, fused_tokens(n, n_loc_max), false, any));
}

hipError_t launch_split(const SplitPlan& p, const SplitArgs& a, int dtype, hipStream_t st) {
    if (p.grid_x <= 0 || p.grid_y <= 0 || p.grid_z <= 0) return hipSuccess;
    if (p.kernel == kMfma16) return launch_split_mfma(p, a, st);
    if (p.kernel == kRows) return launch_split_rows(p, a, st);
    return launch_split_valu(p, a, dtype, a.idx != nullptr, st);
}

}  // namespace lcda

using namespace lcda;

extern "C" {

const char* lcda_last_error(void) { return g_err; }

const char* lcda_version(void) { return "0.1.0"; }

int lcda_set_tuning(const char* key, int64_t value) {
    if (!key) return fail(LCDA_EINVAL, "lcda_set_tuning: key is NULL");
    if (value < 0) return fail(LCDA_EINVAL, "lcda_set_tuning: %s = %lld < 0", key, (long long)value);
    Tuning& t = tuning();
    const bool wgs_ok = value > 0 && value <= kMaxTargetWgs;   // the workspace sizes assume at most this
    if (!strcmp(key, "dense_wgs") && wgs_ok) t.dense_wgs = value;
    else if (!strcmp(key, "dense_wgs_nt4") && wgs_ok) t.dense_wgs_nt4 = value;
    else if (!strcmp(key, "valu_wgs") && wgs_ok) t.valu_wgs = value;
    else if (!strcmp(key, "gather_wgs") && wgs_ok) t.gather_wgs = value;
    else if (!strcmp(key, "gather_waves") && (value == 4 || value == 8 || value == 16)) t.gather_waves = value;
    else if (!strcmp(key, "rows_wgs") && wgs_ok) t.rows_wgs = value;
    else if (!strcmp(key, "rows_wgs_single") && wgs_ok) t.rows_wgs_single = value;
    else if (!strcmp(key, "rows_kernel") && value <= 1) t.rows_kernel = value;
    else if (!strcmp(key, "rows_variant") && value <= 8) t.rows_variant = value;
    else if (!strcmp(key, "direct_blocks")) t.direct_blocks = value;
    else if (!strcmp(key, "dense_variant") && value <= 4) t.dense_variant = value;
    else if (!strcmp(key, "gather_variant") && value <= 1) t.gather_variant = value;
    else if (!strcmp(key, "topk_subs") && value <= 64) t.topk_subs = value;
    else if (!strcmp(key, "topk_wgs") && value > 0) t.topk_wgs = value;
    else if (!strcmp(key, "topk_kernel") && value <= 1) t.topk_kernel = value;
    else if (!strcmp(key, "topk_spin") && value <= (1 << 20)) t.topk_spin = value;
    else if (!strcmp(key, "sparse_fused") && value <= 1) t.sparse_fused = value;
    else if (!strcmp(key, "wide_chunk") && (value == 0 || (value % 4096 == 0 && value <= kWideMaxL))) g_wide_chunk = value;
    else return fail(LCDA_EINVAL, "lcda_set_tuning: unknown key or value for '%s'", key);
    return LCDA_OK;
}

int64_t lcda_get_tuning(const char* key) {
    if (!key) return -1;
    const Tuning& t = tuning();
    if (!strcmp(key, "dense_wgs")) return t.dense_wgs;
    if (!strcmp(key, "dense_wgs_nt4")) return t.dense_wgs_nt4;
    if (!strcmp(key, "valu_wgs")) return t.valu_wgs;
    if (!strcmp(key, "gather_wgs")) return t.gather_wgs;
    if (!strcmp(key, "gather_waves")) return t.gather_waves;
    if (!strcmp(key, "rows_wgs")) return t.rows_wgs;
    if (!strcmp(key, "rows_wgs_single")) return t.rows_wgs_single;
    if (!strcmp(key, "rows_kernel")) return t.rows_kernel;
    if (!strcmp(key, "rows_variant")) return t.rows_variant;
    if (!strcmp(key, "direct_blocks")) return t.direct_blocks;
    if (!strcmp(key, "dense_variant")) return t.dense_variant;
    if (!strcmp(key, "gather_variant")) return t.gather_variant;
    if (!strcmp(key, "topk_subs")) return t.topk_subs;
    if (!strcmp(key, "topk_wgs")) return t.topk_wgs;
    if (!strcmp(key, "topk_kernel")) return t.topk_kernel;
    if (!strcmp(key, "topk_spin")) return t.topk_spin;
    if (!strcmp(key, "sparse_fused")) return t.sparse_fused;
    if (!strcmp(key, "wide_chunk")) return g_wide_chunk;
    return -1;
}

size_t lcda_ws_bytes_cached_attn_lse(int B, int Hq, int Hkv, int d, int64_t n, int64_t kv_batch_stride) {
    if (d != kD || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || n < 0 || n > INT32_MAX) return 0;
    return std::max(split_ws(LCDA_BF16, false, B, Hq, Hkv, n, kv_batch_stride == 0, true),
                    split_ws(LCDA_F32, false, B, Hq, Hkv, n, kv_batch_stride == 0, true));
}

size_t lcda_ws_bytes_lse_merge_local(int B, int Hq, int Hkv, int d, int64_t n_loc_max) {
    return lcda_ws_bytes_cached_attn_lse(B, Hq, Hkv, d, n_loc_max, 1);
}

size_t lcda_ws_bytes_sig_score_topk(int B, int Hq, int Hkv, int64_t n) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || n < 0 || n > INT32_MAX) return 0;
    return topk_layout(B, Hq, Hkv, n).bytes;
}

size_t lcda_ws_bytes_gather_attn(int B, int Hq, int Hkv, int d, int64_t cap) {
    if (d != kD || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || cap < 0 || cap > INT32_MAX) return 0;
    return split_ws(LCDA_BF16, true, B, Hq, Hkv, cap, false, true);
}

static int cached_attn_lse_impl(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int d,
                                int64_t n, int64_t kv_batch_stride, int dtype, float* out, float* alpha,
                                const Scratch& sc, void* stream) {
    static const char* fn = "cached_attn_lse";
    void* ws = sc.ws;
    const size_t ws_bytes = sc.bytes;
    RETURN_IF(check_heads(fn, B, Hq, Hkv, d));
    RETURN_IF(check_dtype(fn, dtype));
    RETURN_IF(check_n(fn, "n", n));
    RETURN_IF(check_kv_stride(fn, kv_batch_stride, Hkv, n, dtype));
    const bool work = B > 0;
    RETURN_IF(check_ptr(fn, "q", q, work));
    RETURN_IF(check_ptr(fn, "k", k, work && n > 0));
    RETURN_IF(check_ptr(fn, "v", v, work && n > 0));
    RETURN_IF(check_ptr(fn, "out", out, work));
    RETURN_IF(check_ptr(fn, "alpha", alpha, work));
    RETURN_IF(check_ptr(fn, "ws", ws, false));
    const bool shared = kv_batch_stride == 0;
    const SplitPlan p = plan_split(dtype, false, B, Hq, Hkv, n, shared);
    const PartialLayout lay = partial_layout(B, Hq, p.splits, sc.ctr == nullptr);
    if (!work) return LCDA_OK;
    if (!ws || ws_bytes < lay.bytes)
        return fail(LCDA_EWORKSPACE, "%s: workspace %zu bytes < %zu required", fn, ws_bytes, lay.bytes);

    SplitArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kv_batch_stride = kv_batch_stride;
    a.n = n;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.shared = shared ? 1 : 0;
    a.rows = shared ? B * a.G : a.G;
    a.row_groups = p.row_groups;
    a.splits = p.splits;
    a.blocks_per_split = p.blocks_per_split;
    a.ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.ml_off);
    a.acc = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.acc_off);
    a.ctr = counters_at(sc, lay);
    a.scale_log2 = kLog2e / sqrtf((float)kD);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(fn, p, a, dtype, B * Hq, out, alpha, nullptr, nullptr, st);
}

int cached_attn_lse(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int d, int64_t n,
                    int64_t kv_batch_stride, int dtype, float* out, float* alpha, void* ws, size_t ws_bytes,
                    void* stream) {
    return cached_attn_lse_impl(q, k, v, B, Hq, Hkv, d, n, kv_batch_stride, dtype, out, alpha,
                                Scratch{ws, ws_bytes, nullptr}, stream);
}

static int lse_merge_local_impl(const void* q, const float* a_in, const float* alpha_in, const void* k_loc,
                                const void* v_loc, const int32_t* n_loc, int64_t n_loc_max, int B, int Hq, int Hkv,
                                int d, int dtype, float* out, float* alpha_out, const Scratch& sc, void* stream) {
    static const char* fn = "lse_merge_local";
    void* ws = sc.ws;
    const size_t ws_bytes = sc.bytes;
    RETURN_IF(check_heads(fn, B, Hq, Hkv, d));
    RETURN_IF(check_dtype(fn, dtype));
    RETURN_IF(check_n(fn, "n_loc_max", n_loc_max));
    const bool work = B > 0;
    RETURN_IF(check_ptr(fn, "q", q, work));
    RETURN_IF(check_ptr(fn, "a_in", a_in, work));
    RETURN_IF(check_ptr(fn, "alpha_in", alpha_in, work));
    RETURN_IF(check_ptr(fn, "k_loc", k_loc, work && n_loc_max > 0));
    RETURN_IF(check_ptr(fn, "v_loc", v_loc, work && n_loc_max > 0));
    RETURN_IF(check_ptr(fn, "n_loc", n_loc, false));
    RETURN_IF(check_ptr(fn, "out", out, work));
    RETURN_IF(check_ptr(fn, "alpha_out", alpha_out, false));
    RETURN_IF(check_ptr(fn, "ws", ws, false));
    if (work && (const void*)out == (const void*)a_in) return fail(LCDA_EINVAL, "%s: out aliases a_in", fn);
    const SplitPlan p = plan_split(dtype, false, B, Hq, Hkv, n_loc_max, false);
    const PartialLayout lay = partial_layout(B, Hq, p.splits, sc.ctr == nullptr);
    if (!work) return LCDA_OK;
    if (!ws || ws_bytes < lay.bytes)
        return fail(LCDA_EWORKSPACE, "%s: workspace %zu bytes < %zu required", fn, ws_bytes, lay.bytes);

    SplitArgs a{};
    a.q = q;
    a.k = k_loc;
    a.v = v_loc;
    a.kv_batch_stride = (int64_t)Hkv * n_loc_max * kD;
    a.n = n_loc_max;
    a.n_b = n_loc;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.shared = 0;
    a.rows = a.G;
    a.row_groups = p.row_groups;
    a.splits = p.splits;
    a.blocks_per_split = p.blocks_per_split;
    a.ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.ml_off);
    a.acc = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.acc_off);
    a.ctr = counters_at(sc, lay);
    a.scale_log2 = kLog2e / sqrtf((float)kD);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(fn, p, a, dtype, B * Hq, out, alpha_out, a_in, alpha_in, st);
}

int lse_merge_local(const void* q, const float* a_in, const float* alpha_in, const void* k_loc,
                    const void* v_loc, const int32_t* n_loc, int64_t n_loc_max, int B, int Hq, int Hkv, int d,
                    int dtype, float* out, float* alpha_out, void* ws, size_t ws_bytes, void* stream) {
    return lse_merge_local_impl(q, a_in, alpha_in, k_loc, v_loc, n_loc, n_loc_max, B, Hq, Hkv, d, dtype, out,
                                alpha_out, Scratch{ws, ws_bytes, nullptr}, stream);
}

// Fused decode step: one split pass over the unified token range (cache, then
// the row's local tokens), then one combine.  A document shared by many rows
// runs the 64-row split pass with the local tokens as extra per-row blocks.
// Falls back to the two calls when no fused form applies (fp32, doc-only
// outputs requested, a shared document read by 16 rows or fewer).
size_t lcda_ws_bytes_dense_decode_step(int B, int Hq, int Hkv, int d, int64_t n, int64_t kv_batch_stride,
                                       int64_t n_loc_max) {
    if (d != kD || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || n < 0 || n > INT32_MAX || n_loc_max < 0 ||
        fused_tokens(n, n_loc_max) > INT32_MAX)
        return 0;
    // Whichever form a call takes (any dtype, with or without a_doc), under any accepted knobs.
    size_t need = 0;
    for (int dt : {LCDA_BF16, LCDA_F32})
        for (int a_doc = 0; a_doc <= 1; ++a_doc)
            need = std::max(need, dense_step_ws(dt, B, Hq, Hkv, n, kv_batch_stride, n_loc_max, a_doc != 0, true));
    return need;
}

}  // extern "C"

namespace lcda {

int dense_decode_step_impl(const void* q, const void* k, const void* v, int64_t kv_batch_stride, int64_t n,
                           const void* k_loc, const void* v_loc, const int32_t* n_loc, int64_t n_loc_max, int B,
                           int Hq, int Hkv, int d, int dtype, float* out, float* alpha_out, float* a_doc,
                           float* alpha_doc, void* ws, size_t ws_bytes, unsigned long long* ctr, void* stream) {
    static const char* fn = "dense_decode_step";
    const Scratch sc{ws, ws_bytes, ctr};
    RETURN_IF(check_heads(fn, B, Hq, Hkv, d));
    RETURN_IF(check_dtype(fn, dtype));
    RETURN_IF(check_n(fn, "n", n));
    RETURN_IF(check_n(fn, "n_loc_max", n_loc_max));
    RETURN_IF(check_n(fn, "n + n_loc_max (cache padded to 32)", fused_tokens(n, n_loc_max)));
    RETURN_IF(check_kv_stride(fn, kv_batch_stride, Hkv, n, dtype));
    const bool work = B > 0;
    RETURN_IF(check_ptr(fn, "q", q, work));
    RETURN_IF(check_ptr(fn, "k", k, work && n > 0));
    RETURN_IF(check_ptr(fn, "v", v, work && n > 0));
    RETURN_IF(check_ptr(fn, "k_loc", k_loc, work && n_loc_max > 0));
    RETURN_IF(check_ptr(fn, "v_loc", v_loc, work && n_loc_max > 0));
    RETURN_IF(check_ptr(fn, "n_loc", n_loc, false));
    RETURN_IF(check_ptr(fn, "out", out, work));
    RETURN_IF(check_ptr(fn, "alpha_out", alpha_out, false));
    RETURN_IF(check_ptr(fn, "a_doc", a_doc, false));
    RETURN_IF(check_ptr(fn, "alpha_doc", alpha_doc, false));
    RETURN_IF(check_ptr(fn, "ws", ws, false));
    if ((a_doc == nullptr) != (alpha_doc == nullptr))
        return fail(LCDA_EINVAL, "%s: a_doc and alpha_doc must both be given or both be NULL", fn);
    const size_t need = dense_step_ws(dtype, B, Hq, Hkv, n, kv_batch_stride, n_loc_max, a_doc != nullptr, false);
    if (!work) return LCDA_OK;
    if (!ws || ws_bytes < need)
        return fail(LCDA_EWORKSPACE, "%s: workspace %zu bytes < %zu required", fn, ws_bytes, need);
    const bool shared = kv_batch_stride == 0 && B > 1;
    if (shared && dtype == LCDA_BF16 && a_doc == nullptr && n > 0 && n_loc_max > 0) {
        // A document shared by many rows: the 64-row split pass also takes each
        // row's local tokens (as extra blocks seen by that row only), then one
        // combine.
        const SplitPlan p = plan_split(dtype, false, B, Hq, Hkv, n, true);
        if (p.kernel == kRows) {
            const PartialLayout lay = partial_layout(B, Hq, p.splits, ctr == nullptr);
            SplitArgs a{};
            a.q = q;
            a.k = k;
            a.v = v;
            a.kv_batch_stride = 0;
            a.n = n;
            a.k2 = k_loc;
            a.v2 = v_loc;
            a.n2 = n_loc_max;
            a.kv2_batch_stride = (int64_t)Hkv * n_loc_max * kD;
            a.n2_b = n_loc;
            a.B = B;
            a.Hq = Hq;
            a.Hkv = Hkv;
            a.G = Hq / Hkv;
            a.shared = 1;
            a.rows = B * a.G;
            a.row_groups = p.row_groups;
            a.splits = p.splits;
            a.blocks_per_split = p.blocks_per_split;
            a.ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.ml_off);
            a.acc = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.acc_off);
            a.ctr = counters_at(sc, lay);
            a.scale_log2 = kLog2e / sqrtf((float)kD);
            return finish(fn, p, a, dtype, B * Hq, out, alpha_out, nullptr, nullptr,
                          static_cast<hipStream_t>(stream));
        }
    }
    if (dtype != LCDA_BF16 || shared || a_doc != nullptr || n == 0 || tuning().dense_variant == 4) {
        // Two-call form: cached_attn_lse, then lse_merge_local on its result.
        char* w = static_cast<char*>(ws);
        const size_t w1 = split_ws(dtype, false, B, Hq, Hkv, n, kv_batch_stride == 0, false);
        const size_t w2 = split_ws(dtype, false, B, Hq, Hkv, n_loc_max, false, false);
        float* A = a_doc;
        float* al = alpha_doc;
        if (!A) {
            A = reinterpret_cast<float*>(w + w1 + w2);
            al = A + (size_t)B * Hq * kD;
        }
        RETURN_IF(cached_attn_lse_impl(q, k, v, B, Hq, Hkv, d, n, kv_batch_stride, dtype, A, al,
                                       Scratch{w, w1, ctr}, stream));
        return lse_merge_local_impl(q, A, al, k_loc, v_loc, n_loc, n_loc_max, B, Hq, Hkv, d, dtype, out, alpha_out,
                                    Scratch{w + w1, w2, ctr}, stream);
    }
    const SplitPlan p = plan_split(dtype, false, B, Hq, Hkv, fused_tokens(n, n_loc_max), false);
    const PartialLayout lay = partial_layout(B, Hq, p.splits, ctr == nullptr);
    SplitArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kv_batch_stride = kv_batch_stride == 0 ? 0 : kv_batch_stride;
    a.n = n;
    a.k2 = k_loc;
    a.v2 = v_loc;
    a.n_c = n;
    a.n2 = n_loc_max;
    a.kv2_batch_stride = (int64_t)Hkv * n_loc_max * kD;
    a.n2_b = n_loc;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.shared = 0;
    a.rows = a.G;
    a.row_groups = p.row_groups;
    a.splits = p.splits;
    a.blocks_per_split = p.blocks_per_split;
    a.ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.ml_off);
    a.acc = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.acc_off);
    a.ctr = counters_at(sc, lay);
    a.scale_log2 = kLog2e / sqrtf((float)kD);
    return finish(fn, p, a, dtype, B * Hq, out, alpha_out, nullptr, nullptr, static_cast<hipStream_t>(stream));
}

}  // namespace lcda

extern "C" {

int dense_decode_step(const void* q, const void* k, const void* v, int64_t kv_batch_stride, int64_t n,
                      const void* k_loc, const void* v_loc, const int32_t* n_loc, int64_t n_loc_max, int B, int Hq,
                      int Hkv, int d, int dtype, float* out, float* alpha_out, float* a_doc, float* alpha_doc,
                      void* ws, size_t ws_bytes, void* stream) {
    return dense_decode_step_impl(q, k, v, kv_batch_stride, n, k_loc, v_loc, n_loc, n_loc_max, B, Hq, Hkv, d, dtype,
                                  out, alpha_out, a_doc, alpha_doc, ws, ws_bytes, nullptr, stream);
}

// sig_score_topk and sig_score_topk_q.  enc: q, R and bits are given, and the
// query codes are encoded into q_sigs by the histogram pass.
static int topk_impl(const char* fn, const uint32_t* key_sigs, uint32_t* q_sigs, const void* q, int q_dtype, const float* R,
              int bits, bool enc, int B, int Hq, int Hkv, int64_t n, int64_t m, int64_t n_sink, int64_t n_recent,
              int32_t* idx, int64_t cap, int32_t* count, int8_t* scores, void* ws, size_t ws_bytes, void* stream) {
    if (B < 0) return fail(LCDA_EINVAL, "%s: B = %d < 0", fn, B);
    if (Hq <= 0 || Hkv <= 0) return fail(LCDA_EINVAL, "%s: Hq = %d, Hkv = %d must be positive", fn, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(LCDA_EINVAL, "%s: Hq = %d is not a multiple of Hkv = %d", fn, Hq, Hkv);
    if (Hq / Hkv > 8) return fail(LCDA_EUNSUPPORTED, "%s: more than 8 query heads per KV head", fn);
    RETURN_IF(check_n(fn, "n", n));
    if (m < 0 || n_sink < 0 || n_recent < 0)
        return fail(LCDA_EINVAL, "%s: m, n_sink and n_recent must be >= 0", fn);
    if (m > INT32_MAX || n_sink > INT32_MAX || n_recent > INT32_MAX)   // before the sum below: no overflow
        return fail(LCDA_EINVAL, "%s: m, n_sink and n_recent must be <= INT32_MAX", fn);
    if (cap < 0 || cap > INT32_MAX) return fail(LCDA_EINVAL, "%s: cap = %lld out of range", fn, (long long)cap);
    const int64_t need = (m + n_sink + n_recent < n) ? m + n_sink + n_recent : n;
    if (cap < need)
        return fail(LCDA_EINVAL, "%s: cap = %lld < min(n, m + n_sink + n_recent) = %lld", fn, (long long)cap,
                    (long long)need);
    const bool work = B > 0;
    RETURN_IF(check_ptr(fn, "key_sigs", key_sigs, work && n > 0));
    RETURN_IF(check_ptr(fn, "q_sigs", q_sigs, work));
    if (enc) {
        RETURN_IF(check_dtype(fn, q_dtype));
        RETURN_IF(check_ptr(fn, "q", q, work));
        RETURN_IF(check_ptr(fn, "R", R, work));
        if (bits < 1 || bits > 32) return fail(LCDA_EINVAL, "%s: bits = %d outside 1 .. 32", fn, bits);
    }
    RETURN_IF(check_ptr(fn, "idx", idx, work && cap > 0));
    RETURN_IF(check_ptr(fn, "count", count, work));
    RETURN_IF(check_ptr(fn, "scores", scores, false));
    RETURN_IF(check_ptr(fn, "ws", ws, false));
    const TopkLayout lay = topk_layout(B, Hq, Hkv, n);
    if (!work) return LCDA_OK;
    if (!ws || ws_bytes < lay.bytes)
        return fail(LCDA_EWORKSPACE, "%s: workspace %zu bytes < %zu required", fn, ws_bytes, lay.bytes);
    TopkArgs a{};
    a.key_sigs = key_sigs;
    a.q_sigs = q_sigs;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.n = n;
    a.m = m;
    a.n_sink = n_sink;
    a.n_recent = n_recent;
    a.cap = cap;
    a.idx = idx;
    a.count = count;
    a.scores = scores;
    char* w = static_cast<char*>(ws);
    // One launch with the distances in LDS where the grid fits the device one
    // workgroup per CU; otherwise the chunked passes.
    const int part = (n > 0 && tuning().topk_kernel == 1) ? topk_unit_part(n, B * Hkv, a.G, device_cus()) : 0;
    if (part > 0) {
        a.parts = (int)ceil_div(n, part);
        a.part_len = part;
        a.spin_max = (int)tuning().topk_spin;
        set_unit_ws(a, w, lay);
        a.chunks = 1;
    } else {
        a.hist = reinterpret_cast<uint32_t*>(w);
        a.chunk_len = topk_chunk_len(n, B * Hkv);
        a.chunks = n > 0 ? (int)ceil_div(n, a.chunk_len) : 0;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (enc && a.chunks == 0) {   // no positions: the codes still come back, from the encoder
        EncodeArgs e{};
        e.x = q;
        e.bf16 = q_dtype == LCDA_BF16;
        e.groups = 1;
        e.rows_per_group = (int64_t)B * Hq;
        e.x_group_stride = 0;
        e.R = R;
        e.bits = bits;
        e.codes = q_sigs;
        e.codes_group_stride = 0;
        RETURN_IF(hip_status(fn, launch_sig_encode(e, st)));
    } else if (enc) {
        a.q = q;
        a.q_bf16 = q_dtype == LCDA_BF16;
        a.R = R;
        a.bits = bits;
        a.q_codes = q_sigs;
    }
    return hip_status(fn, launch_topk(a, st));
}

int sig_score_topk(const uint32_t* key_sigs, const uint32_t* q_sigs, int B, int Hq, int Hkv, int64_t n,
                   int64_t m, int64_t n_sink, int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                   int8_t* scores, void* ws, size_t ws_bytes, void* stream) {
    return topk_impl("sig_score_topk", key_sigs, const_cast<uint32_t*>(q_sigs), nullptr, 0, nullptr, 0, false, B, Hq,
                     Hkv, n, m, n_sink, n_recent, idx, cap, count, scores, ws, ws_bytes, stream);
}

int sig_score_topk_q(const uint32_t* key_sigs, const void* q, int q_dtype, const float* R, int bits, int B, int Hq,
                     int Hkv, int64_t n, int64_t m, int64_t n_sink, int64_t n_recent, int32_t* idx, int64_t cap,
                     int32_t* count, int8_t* scores, uint32_t* q_sigs, void* ws, size_t ws_bytes, void* stream) {
    return topk_impl("sig_score_topk_q", key_sigs, q_sigs, q, q_dtype, R, bits, true, B, Hq, Hkv, n, m, n_sink,
                     n_recent, idx, cap, count, scores, ws, ws_bytes, stream);
}

// Workspace of sig_score_topk_w: distance bytes ([B, Hkv, groups][n][HG]: at
// most 2 B Hq n bytes, as HG <= 2G - 1 for G <= 8 and groups * 8 < 2G above),
// per-chunk histograms (rows padded to 16 bytes, sized for the widest code),
// per-chunk offsets and per-row thresholds.  W = 1 may run the one-word kernel
// instead, in the same workspace, which is sized for that too (its layout only
// grows with Hkv, so Hkv = Hq bounds it).
struct WideLayout {
    size_t dist, hist, rec, rowrec, bytes;
    int64_t n16, nc_max;
};
constexpr int kWideBinsP = 520;   // 513 bins padded to a multiple of 8
WideLayout wide_layout(int B, int Hq, int64_t n) {
    WideLayout l{};
    const size_t rows = (size_t)B * Hq;
    l.n16 = (n + 15) / 16 * 16;
    l.nc_max = std::max<int64_t>(1, ceil_div(n, kWideMinL));
    l.dist = 0;
    l.hist = l.dist + round_up(2 * rows * (size_t)l.n16);
    l.rec = l.hist + round_up(3 * rows * (size_t)l.nc_max * kWideBinsP * sizeof(uint16_t));
    l.rowrec = l.rec + round_up(rows * (size_t)l.nc_max * 2 * sizeof(uint32_t));
    l.bytes = l.rowrec + round_up(rows * 2 * sizeof(int32_t));
    return l;
}

size_t lcda_ws_bytes_sig_score_topk_w(int B, int Hq, int64_t n) {
    if (B < 0 || Hq <= 0 || n < 0 || n > INT32_MAX) return 0;
    return std::max(wide_layout(B, Hq, n).bytes, topk_layout(B, Hq, Hq, n).bytes);
}

int sig_score_topk_w(const uint32_t* key_sigs, const uint32_t* q_sigs, int W, int B, int Hq, int Hkv, int64_t n,
                     int64_t m, int64_t n_sink, int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count,
                     int16_t* scores, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "sig_score_topk_w";
    if (W != 1 && W != 2 && W != 4 && W != 8 && W != 16)
        return fail(LCDA_EUNSUPPORTED, "%s: W = %d words (1, 2, 4, 8 or 16 supported)", fn, W);
    if (B < 0) return fail(LCDA_EINVAL, "%s: B = %d < 0", fn, B);
    if (Hq <= 0 || Hkv <= 0) return fail(LCDA_EINVAL, "%s: Hq = %d, Hkv = %d must be positive", fn, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(LCDA_EINVAL, "%s: Hq = %d is not a multiple of Hkv = %d", fn, Hq, Hkv);
    RETURN_IF(check_n(fn, "n", n));
    if (m < 0 || n_sink < 0 || n_recent < 0)
        return fail(LCDA_EINVAL, "%s: m, n_sink and n_recent must be >= 0", fn);
    if (m > INT32_MAX || n_sink > INT32_MAX || n_recent > INT32_MAX)   // before the sum below: no overflow
        return fail(LCDA_EINVAL, "%s: m, n_sink and n_recent must be <= INT32_MAX", fn);
    if (cap < 0 || cap > INT32_MAX) return fail(LCDA_EINVAL, "%s: cap = %lld out of range", fn, (long long)cap);
    const int64_t need = (m + n_sink + n_recent < n) ? m + n_sink + n_recent : n;
    if (cap < need)
        return fail(LCDA_EINVAL, "%s: cap = %lld < min(n, m + n_sink + n_recent) = %lld", fn, (long long)cap,
                    (long long)need);
    const bool work = B > 0;
    RETURN_IF(check_ptr(fn, "key_sigs", key_sigs, work && n > 0));
    RETURN_IF(check_ptr(fn, "q_sigs", q_sigs, work));
    RETURN_IF(check_ptr(fn, "idx", idx, work && cap > 0));
    RETURN_IF(check_ptr(fn, "count", count, work));
    RETURN_IF(check_ptr(fn, "scores", scores, false));
    RETURN_IF(check_ptr(fn, "ws", ws, false));
    if (!work) return LCDA_OK;
    const size_t need_ws = lcda_ws_bytes_sig_score_topk_w(B, Hq, n);
    if (!ws || ws_bytes < need_ws)
        return fail(LCDA_EWORKSPACE, "%s: workspace %zu bytes < %zu required", fn, ws_bytes, need_ws);
    // One word without scores: the one-word kernel computes this very selection.
    if (W == 1 && !scores && Hq / Hkv <= 8)
        return topk_impl(fn, key_sigs, const_cast<uint32_t*>(q_sigs), nullptr, 0, nullptr, 0, false, B, Hq, Hkv, n, m,
                         n_sink, n_recent, idx, cap, count, nullptr, ws, ws_bytes, stream);
    WideArgs a{};
    a.key_sigs = key_sigs;
    a.q_sigs = q_sigs;
    a.W = W;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.n = n;
    a.m = m;
    a.n_sink = n_sink;
    a.n_recent = n_recent;
    a.cap = cap;
    a.idx = idx;
    a.count = count;
    a.scores = scores;
    a.HG = wide_group(a.G);
    a.ng = (a.G + a.HG - 1) / a.HG;
    const WideLayout l = wide_layout(B, Hq, n);
    // Chunks: as many as make the histogram and compaction grids fill the
    // workgroup slots of the device in whole rounds (one round where the
    // chunk length allows), at most 32 per head where that suffices (the
    // select pass stages 32 chunks at a time), never more than the workspace
    // holds (n / kWideMinL) nor longer than kWideMaxL positions; the length
    // is a whole number of histogram-loop turns and compaction tiles.
    const int64_t units = (int64_t)B * Hkv * a.ng;
    const int64_t slots = (int64_t)std::max(1, wide_slots_per_cu(W, a.HG)) * std::max(1, device_cus());
    const int64_t nc_min = ceil_div(n, kWideMaxL);
    int64_t want = 1;
    for (int64_t k = 1;; ++k) {
        want = std::max<int64_t>(1, k * slots / units);
        if (want >= nc_min) break;
    }
    if (want > 32) want = std::max<int64_t>(32, nc_min);
    want = std::min(want, l.nc_max);
    const int64_t gran = wide_granule(W);   // divides kWideMaxL
    a.L = n > 0 ? ceil_div(ceil_div(n, want), gran) * gran : gran;
    if (g_wide_chunk > 0) a.L = std::max(g_wide_chunk, ceil_div(ceil_div(n, l.nc_max), gran) * gran);
    a.nc = ceil_div(n, a.L);
    a.dstride = l.n16 * a.HG;
    a.vec = (n * W) % 4 == 0;   // key_sigs is 16-byte aligned (checked above)
    char* base = static_cast<char*>(ws);
    a.dist = reinterpret_cast<uint8_t*>(base + l.dist);
    a.hist = reinterpret_cast<uint16_t*>(base + l.hist);
    a.rec = reinterpret_cast<uint32_t*>(base + l.rec);
    a.rowrec = reinterpret_cast<int32_t*>(base + l.rowrec);
    return hip_status(fn, launch_topk_wide(a, static_cast<hipStream_t>(stream)));
}

int sig_encode(const void* x, int dtype, int64_t groups, int64_t rows_per_group, int64_t x_group_stride,
               const float* R, int bits, uint32_t* codes, int64_t codes_group_stride, void* stream) {
    static const char* fn = "sig_encode";
    RETURN_IF(check_dtype(fn, dtype));
    if (groups < 0 || rows_per_group < 0)
        return fail(LCDA_EINVAL, "%s: groups = %lld, rows_per_group = %lld must be >= 0", fn, (long long)groups,
                    (long long)rows_per_group);
    if (bits < 1 || bits > 32) return fail(LCDA_EINVAL, "%s: bits = %d outside 1 .. 32", fn, bits);
    const bool work = groups > 0 && rows_per_group > 0;
    if (work && rows_per_group > INT32_MAX / groups)   // rows above INT32_MAX: beyond any grid here
        return fail(LCDA_EUNSUPPORTED, "%s: groups * rows_per_group = %lld * %lld exceeds INT32_MAX rows", fn,
                    (long long)groups, (long long)rows_per_group);
    if (work && groups > 1 && (x_group_stride < rows_per_group * kD || codes_group_stride < rows_per_group))
        return fail(LCDA_EINVAL, "%s: group strides overlap the rows (x %lld < %lld or codes %lld < %lld)", fn,
                    (long long)x_group_stride, (long long)(rows_per_group * kD), (long long)codes_group_stride,
                    (long long)rows_per_group);
    if (x_group_stride < 0 || x_group_stride % 8 != 0 || codes_group_stride < 0)
        return fail(LCDA_EINVAL, "%s: x_group_stride must be a non-negative multiple of 8, codes_group_stride >= 0",
                    fn);
    RETURN_IF(check_ptr(fn, "x", x, work));
    RETURN_IF(check_ptr(fn, "R", R, work));
    if (work && !codes) return fail(LCDA_EINVAL, "%s: codes is NULL", fn);
    if (codes && reinterpret_cast<uintptr_t>(codes) % 4 != 0)
        return fail(LCDA_EINVAL, "%s: codes is not 4-byte aligned", fn);
    if (!work) return LCDA_OK;
    EncodeArgs e{};
    e.x = x;
    e.bf16 = dtype == LCDA_BF16;
    e.groups = groups;
    e.rows_per_group = rows_per_group;
    e.x_group_stride = x_group_stride;
    e.R = R;
    e.bits = bits;
    e.codes = codes;
    e.codes_group_stride = codes_group_stride;
    return hip_status(fn, launch_sig_encode(e, static_cast<hipStream_t>(stream)));
}

int gather_attn(const void* q, const void* k, const void* v, int64_t kv_batch_stride, const int32_t* idx,
                const int32_t* count, int64_t cap, int B, int Hq, int Hkv, int d, int64_t n, int dtype, float* out,
                float* alpha, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "gather_attn";
    RETURN_IF(check_heads(fn, B, Hq, Hkv, d));
    RETURN_IF(check_dtype(fn, dtype));
    RETURN_IF(check_n(fn, "n", n));
    RETURN_IF(check_n(fn, "cap", cap));
    RETURN_IF(check_kv_stride(fn, kv_batch_stride, Hkv, n, dtype));
    const bool work = B > 0;
    RETURN_IF(check_ptr(fn, "q", q, work));
    RETURN_IF(check_ptr(fn, "k", k, work && n > 0));
    RETURN_IF(check_ptr(fn, "v", v, work && n > 0));
    RETURN_IF(check_ptr(fn, "idx", idx, work && cap > 0));
    RETURN_IF(check_ptr(fn, "count", count, work));
    RETURN_IF(check_ptr(fn, "out", out, work));
    RETURN_IF(check_ptr(fn, "alpha", alpha, false));
    RETURN_IF(check_ptr(fn, "ws", ws, false));
    const SplitPlan p = plan_split(dtype, true, B, Hq, Hkv, cap, false);
    const PartialLayout lay = partial_layout(B, Hq, p.splits);
    if (!work) return LCDA_OK;
    if (!ws || ws_bytes < lay.bytes)
        return fail(LCDA_EWORKSPACE, "%s: workspace %zu bytes < %zu required", fn, ws_bytes, lay.bytes);
    SplitArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.kv_batch_stride = kv_batch_stride;
    a.n = n;
    a.idx = idx;
    a.count = count;
    a.cap = cap;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.shared = kv_batch_stride == 0 ? 1 : 0;
    a.rows = 1;
    a.row_groups = 1;
    a.splits = p.splits;
    a.blocks_per_split = p.blocks_per_split;
    a.ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + lay.ml_off);
    a.acc = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.acc_off);
    a.ctr = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + lay.ctr_off);
    a.scale_log2 = kLog2e / sqrtf((float)kD);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(fn, p, a, dtype, B * Hq, out, alpha, nullptr, nullptr, st);
}

// Fused sparse decode step: SCORE + TOPK + GATHER-ATT in one launch where the
// one-launch TOPK form applies (every part of the launch resident at once,
// G <= 4); otherwise sig_score_topk then gather_attn.  Workspace: the TOPK
// layout, then the merge counters and the parts' partial states.
struct SparseLayout {
    size_t bar2_off, pml_off, pacc_off, bytes;
};

static SparseLayout sparse_layout(int B, int Hq, int Hkv, int64_t n) {
    SparseLayout l;
    const size_t rows = (size_t)B * Hq, units = (size_t)B * Hkv;
    const size_t max_parts = (size_t)std::min<int64_t>(64, std::max<int64_t>(1, (n + 4095) / 4096));
    l.bar2_off = topk_layout(B, Hq, Hkv, n).bytes;
    l.pml_off = l.bar2_off + round_up(units * sizeof(unsigned long long));
    l.pacc_off = l.pml_off + round_up(rows * max_parts * sizeof(float2));
    l.bytes = l.pacc_off + round_up(rows * max_parts * kD * sizeof(float));
    return l;
}

size_t lcda_ws_bytes_sparse_decode_step(int B, int Hq, int Hkv, int d, int64_t n, int64_t cap) {
    if (d != kD || B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || n < 0 || n > INT32_MAX || cap < 0 || cap > INT32_MAX)
        return 0;
    const size_t fused = sparse_layout(B, Hq, Hkv, n).bytes;
    const size_t two = std::max(lcda_ws_bytes_sig_score_topk(B, Hq, Hkv, n), lcda_ws_bytes_gather_attn(B, Hq, Hkv, d, cap));
    return std::max(fused, two);
}

int sparse_decode_step(const uint32_t* key_sigs, const uint32_t* q_sigs, const void* q, const void* k, const void* v,
                       int64_t kv_batch_stride, int B, int Hq, int Hkv, int d, int64_t n, int dtype, int64_t m,
                       int64_t n_sink, int64_t n_recent, int32_t* idx, int64_t cap, int32_t* count, float* out,
                       float* alpha, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "sparse_decode_step";
    RETURN_IF(check_heads(fn, B, Hq, Hkv, d));
    RETURN_IF(check_dtype(fn, dtype));
    RETURN_IF(check_n(fn, "n", n));
    RETURN_IF(check_kv_stride(fn, kv_batch_stride, Hkv, n, dtype));
    if (Hq / Hkv > 8) return fail(LCDA_EUNSUPPORTED, "%s: more than 8 query heads per KV head", fn);
    if (m < 0 || n_sink < 0 || n_recent < 0) return fail(LCDA_EINVAL, "%s: m, n_sink and n_recent must be >= 0", fn);
    if (m > INT32_MAX || n_sink > INT32_MAX || n_recent > INT32_MAX)
        return fail(LCDA_EINVAL, "%s: m, n_sink and n_recent must be <= INT32_MAX", fn);
    if (cap < 0 || cap > INT32_MAX) return fail(LCDA_EINVAL, "%s: cap = %lld out of range", fn, (long long)cap);
    const int64_t need = std::min(n, m + n_sink + n_recent);
    if (cap < need)
        return fail(LCDA_EINVAL, "%s: cap = %lld < min(n, m + n_sink + n_recent) = %lld", fn, (long long)cap,
                    (long long)need);
    const bool work = B > 0;
    RETURN_IF(check_ptr(fn, "key_sigs", key_sigs, work && n > 0));
    RETURN_IF(check_ptr(fn, "q_sigs", q_sigs, work));
    RETURN_IF(check_ptr(fn, "q", q, work));
    RETURN_IF(check_ptr(fn, "k", k, work && n > 0));
    RETURN_IF(check_ptr(fn, "v", v, work && n > 0));
    RETURN_IF(check_ptr(fn, "idx", idx, work && cap > 0));
    RETURN_IF(check_ptr(fn, "count", count, work));
    RETURN_IF(check_ptr(fn, "out", out, work));
    RETURN_IF(check_ptr(fn, "alpha", alpha, false));
    RETURN_IF(check_ptr(fn, "ws", ws, false));
    if (!work) return LCDA_OK;
    const size_t need_ws = lcda_ws_bytes_sparse_decode_step(B, Hq, Hkv, d, n, cap);
    if (!ws || ws_bytes < need_ws)
        return fail(LCDA_EWORKSPACE, "%s: workspace %zu bytes < %zu required", fn, ws_bytes, need_ws);
    const int G = Hq / Hkv;
    const int part = (n > 0 && tuning().topk_kernel == 1 && tuning().sparse_fused == 1)
                         ? topk_unit_part(n, B * Hkv, G, device_cus())
                         : 0;
    if (part == 0) {   // the two calls
        RETURN_IF(sig_score_topk(key_sigs, q_sigs, B, Hq, Hkv, n, m, n_sink, n_recent, idx, cap, count, nullptr, ws,
                                 ws_bytes, stream));
        return gather_attn(q, k, v, kv_batch_stride, idx, count, cap, B, Hq, Hkv, d, n, dtype, out, alpha, ws,
                           ws_bytes, stream);
    }
    const TopkLayout lay = topk_layout(B, Hq, Hkv, n);
    const SparseLayout sl = sparse_layout(B, Hq, Hkv, n);
    char* w = static_cast<char*>(ws);
    TopkArgs a{};
    a.key_sigs = key_sigs;
    a.q_sigs = q_sigs;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.n = n;
    a.m = m;
    a.n_sink = n_sink;
    a.n_recent = n_recent;
    a.cap = cap;
    a.idx = idx;
    a.count = count;
    a.chunks = 1;
    a.parts = (int)ceil_div(n, part);
    a.part_len = part;
    a.spin_max = (int)tuning().topk_spin;
    set_unit_ws(a, w, lay);
    a.gq = q;
    a.gk = k;
    a.gv = v;
    a.kv_batch_stride = kv_batch_stride;
    a.out = out;
    a.alpha = alpha;
    a.bar2 = reinterpret_cast<unsigned long long*>(w + sl.bar2_off);
    a.pml = reinterpret_cast<float2*>(w + sl.pml_off);
    a.pacc = reinterpret_cast<float*>(w + sl.pacc_off);
    a.scale_log2 = kLog2e / sqrtf((float)kD);
    return hip_status(fn, launch_topk_unit(a, dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
