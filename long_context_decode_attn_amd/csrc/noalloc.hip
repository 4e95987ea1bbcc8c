// noalloc.hip - dense_decode_step for callers that cannot allocate: the
// partial states and arrival counters live in a file-scope device array
// instead of a caller-provided workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Its address on a device is looked up once, with that device
// current, through hipGetSymbolAddress; host code never passes the array's
// name itself to a kernel (on the host it is only a stand-in symbol).
//
// Layout of the array: a region that holds only the split pass's arrival
// counters (one 64-bit word per work unit), then the workspace proper.  The
// array starts zeroed; a counter word is either 0 (never used, which the
// arrival replaces by its tagged form) or the (tag, 0) word every call leaves,
// so no call needs to clear anything, and no other data ever lands where a
// counter lives.  Every call on a device shares that device's array: calls
// that overlap on one device (concurrent streams) race.

#include <mutex>

#include "../../include/lcda.h"
#include "common.h"
#include "internal.h"

namespace lcda {

int dense_decode_step_impl(const void* q, const void* k, const void* v, int64_t kv_batch_stride, int64_t n,
                           const void* k_loc, const void* v_loc, const int32_t* n_loc, int64_t n_loc_max, int B,
                           int Hq, int Hkv, int d, int dtype, float* out, float* alpha_out, float* a_doc,
                           float* alpha_doc, void* ws, size_t ws_bytes, unsigned long long* ctr, void* stream);
size_t dense_step_ws(int dtype, int B, int Hq, int Hkv, int64_t n, int64_t kv_batch_stride, int64_t n_loc_max,
                     bool a_doc, bool any);

namespace {

constexpr size_t kCtrBytes = (size_t)kNoallocMaxRows * sizeof(unsigned long long);

__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // scratch's device address, per device (null until looked up)

// scratch's address on the current device, looked up on the first call there.
int scratch_ptr(const char* fn, char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(LCDA_EHIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return set_error(LCDA_EUNSUPPORTED, "%s: device %d beyond the %d supported", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return set_error(LCDA_EHIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                             hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = static_cast<char*>(g_ptr[dev]);
    return LCDA_OK;
}

}  // namespace
}  // namespace lcda

using namespace lcda;

extern "C" {

size_t lcda_noalloc_scratch_bytes(void) { return kNoallocScratchBytes - kCtrBytes; }

int dense_decode_step_noalloc(const void* q, const void* k, const void* v, int64_t kv_batch_stride, int64_t n,
                              const void* k_loc, const void* v_loc, const int32_t* n_loc, int64_t n_loc_max, int B,
                              int Hq, int Hkv, int d, int dtype, float* out, float* alpha_out, void* stream) {
    static const char* fn = "dense_decode_step_noalloc";
    if (B > 0 && Hq > 0 && (int64_t)B * Hq > kNoallocMaxRows)
        return set_error(LCDA_EUNSUPPORTED, "%s: B*Hq = %lld query rows exceed the %d supported", fn,
                         (long long)B * Hq, kNoallocMaxRows);
    // The workspace this call takes under the current knobs (the shape checks come below).
    const bool shapes_ok = d == kD && B >= 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && n >= 0 && n <= INT32_MAX &&
                           n_loc_max >= 0 && n_loc_max <= INT32_MAX && (dtype == LCDA_F32 || dtype == LCDA_BF16);
    const size_t need =
        shapes_ok ? dense_step_ws(dtype, B, Hq, Hkv, n, kv_batch_stride, n_loc_max, false, false) : 0;
    if (need > lcda_noalloc_scratch_bytes())
        return set_error(LCDA_EUNSUPPORTED, "%s: the shapes need %zu bytes of scratch, more than the %zu held", fn,
                         need, lcda_noalloc_scratch_bytes());
    // Every argument check runs first: without a workspace the call returns
    // LCDA_EWORKSPACE only when all else is valid and there is work to do.
    const int v0 = dense_decode_step_impl(q, k, v, kv_batch_stride, n, k_loc, v_loc, n_loc, n_loc_max, B, Hq, Hkv, d,
                                          dtype, out, alpha_out, nullptr, nullptr, nullptr, 0, nullptr, stream);
    if (v0 != LCDA_EWORKSPACE) return v0;
    char* base = nullptr;
    const int s = scratch_ptr(fn, &base);
    if (s != LCDA_OK) return s;
    return dense_decode_step_impl(q, k, v, kv_batch_stride, n, k_loc, v_loc, n_loc, n_loc_max, B, Hq, Hkv, d, dtype,
                                  out, alpha_out, nullptr, nullptr, base + kCtrBytes, lcda_noalloc_scratch_bytes(),
                                  reinterpret_cast<unsigned long long*>(base), stream);
}

}  // extern "C"
