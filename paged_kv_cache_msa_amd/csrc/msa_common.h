// Host-side pieces shared by the library sources: the device form of a cache view, its validation
// and the RoPE inverse frequencies.  Internal to the library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "msa_produce.h"

namespace msa_internal {

constexpr int kHeadDim = 128;

// Device form of an msa_cache_view (element strides; the dim stride is 1).
struct CacheDev {
    uint8_t* data;
    int64_t sp, sh, st;        // element strides (page, head, token)
    const float* scale;        // fp8 only
    int32_t heads;
    int32_t is_bf16;
};


inline bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Validates a cache view of `heads` heads over `num_pages` pages of `page_size` tokens and fills its
// device form.  heads == 0: nothing to check, the descriptor may be NULL.  `vec`: the fused
// producer's layout (16-byte aligned base, strides multiples of 8 elements); otherwise any positive
// strides and a base aligned to the element size.  `span`: if given, receives the bytes from the
// view's base to one past its last element (0 without heads).
inline msa_status check_cache(const msa_cache_view* v, int32_t heads, int32_t page_size, int64_t num_pages, CacheDev* out,
                              bool vec = true, uint64_t* span = nullptr)
{
    std::memset(out, 0, sizeof(*out));
    if (span) *span = 0;
    if (heads == 0) return MSA_OK;
    if (!v || !v->data) return MSA_ERR_NULL_POINTER;
    if (v->num_heads != heads) return MSA_ERR_SHAPE;
    if (v->dtype != MSA_CACHE_FP8_E4M3 && v->dtype != MSA_CACHE_BF16) return MSA_ERR_DTYPE;
    if (v->dtype == MSA_CACHE_FP8_E4M3 && !v->scale) return MSA_ERR_DTYPE;
    if (!aligned(v->data, vec ? 16 : v->dtype == MSA_CACHE_BF16 ? 2 : 1)) return MSA_ERR_ALIGNMENT;
    if (v->dtype == MSA_CACHE_FP8_E4M3 && !aligned(v->scale, 4)) return MSA_ERR_ALIGNMENT;
    const int64_t s[3] = {v->stride_page, v->stride_head, v->stride_token};
    for (int i = 0; i < 3; ++i)
        if (s[i] <= 0 || (vec && s[i] % 8)) return MSA_ERR_STRIDE;
    // Non-overlap: with the dims ordered by stride, each stride must exceed the largest offset
    // the smaller dims can reach.  The walk also yields the largest element offset of the view.
    int64_t ord_s[4] = {1, s[2], s[1], s[0]};
    int64_t ord_e[4] = {kHeadDim, page_size, heads, num_pages};
    for (int i = 1; i < 4; ++i)
        for (int j = i; j > 0 && ord_s[j] < ord_s[j - 1]; --j) {
            const int64_t ts = ord_s[j]; ord_s[j] = ord_s[j - 1]; ord_s[j - 1] = ts;
            const int64_t te = ord_e[j]; ord_e[j] = ord_e[j - 1]; ord_e[j - 1] = te;
        }
    int64_t max_off = 0;
    for (int i = 0; i < 4; ++i) {
        if (ord_e[i] <= 1) continue;
        if (ord_s[i] <= max_off) return MSA_ERR_STRIDE;
        int64_t reach;
        if (__builtin_mul_overflow(ord_s[i], ord_e[i] - 1, &reach) || __builtin_add_overflow(max_off, reach, &max_off))
            return MSA_ERR_OVERFLOW;
    }
    int64_t bytes;
    if (__builtin_mul_overflow(max_off + 1, (int64_t)(v->dtype == MSA_CACHE_BF16 ? 2 : 1), &bytes))
        return MSA_ERR_OVERFLOW;
    if (span) *span = num_pages > 0 ? (uint64_t)bytes : 0;
    out->data = static_cast<uint8_t*>(v->data);
    out->sp = s[0];
    out->sh = s[1];
    out->st = s[2];
    out->scale = v->dtype == MSA_CACHE_FP8_E4M3 ? v->scale : nullptr;   // a bf16 cache's scale is never read
    out->heads = heads;
    out->is_bf16 = v->dtype == MSA_CACHE_BF16;
    return MSA_OK;
}

// ------------------------------------------------------------------ residency of the kernels' operands

// One operand of a launch: the bytes [p, p + bytes) its kernels may touch.
struct Span {
    const void* p;
    uint64_t bytes;
};

// Whether kernels on device `device` may touch [p, p + bytes): the HIP runtime knows the memory, it
// is device memory of that device, managed memory, or pinned host memory mapped at the same
// address, and the range lies inside its allocation (where the runtime reports the allocation's
// extent).  NULL or empty spans pass.  A failed runtime query leaves no error behind for later calls.
inline bool span_resident(const Span& s, int device)
{
    if (!s.p || s.bytes == 0) return true;
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, s.p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    switch (at.type) {
        case hipMemoryTypeDevice:
            if (at.device != device) return false;
            break;
        case hipMemoryTypeManaged:
            break;
        case hipMemoryTypeHost:
            if (at.devicePointer != s.p) return false;
            break;
        default:
            return false;
    }
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(s.p)) != hipSuccess) {
        (void)hipGetLastError();
        return true;      // extent not reported (the kind of memory is already known to be accessible)
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(s.p);
    return q >= b && q - b <= size && s.bytes <= size - (q - b);
}

// The residency check of n spans on the current device; *first_bad = index of the first failing
// span (or -1).
inline msa_status spans_resident(const Span* s, int n, int32_t* first_bad)
{
    if (first_bad) *first_bad = -1;
    int device = -1;
    for (int i = 0; i < n; ++i) {
        if (!s[i].p || s[i].bytes == 0) continue;
        bool ok = true;
        if (device < 0 && hipGetDevice(&device) != hipSuccess) {
            (void)hipGetLastError();
            device = -1;
            ok = false;
        }
        if (!ok || !span_resident(s[i], device)) {
            if (first_bad) *first_bad = i;
            return MSA_ERR_NOT_DEVICE;
        }
    }
    return MSA_OK;
}

// What every launching entry point runs after its argument checks and before its first launch:
// the residency check of its operands, for eager calls.  While `stream` is being captured into a
// graph nothing runs here (no runtime query beyond the capture status), since the captured
// pointers are the caller's to keep alive and valid for every replay.
inline msa_status check_operands(const Span* s, int n, hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return MSA_ERR_LAUNCH;
    }
    if (cs != hipStreamCaptureStatusNone) return MSA_OK;
    return spans_resident(s, n, nullptr);
}

// Bytes of `count` elements of `elem` bytes, saturating (a saturated extent fails the check).
inline uint64_t nbytes(int64_t count, int64_t elem)
{
    if (count <= 0) return 0;
    int64_t b;
    return __builtin_mul_overflow(count, elem, &b) ? UINT64_MAX : (uint64_t)b;
}

// Bytes a row view of `rows` rows of `row_elems` elements at a stride of `stride` elements spans.
inline uint64_t row_bytes(int64_t rows, int64_t stride, int64_t row_elems, int64_t elem)
{
    if (rows <= 0 || row_elems <= 0) return 0;
    int64_t last;
    if (__builtin_mul_overflow(rows - 1, stride, &last) || __builtin_add_overflow(last, row_elems, &last))
        return UINT64_MAX;
    return nbytes(last, elem);
}

// inv_freq_i = 1 / theta^(2i/D) in binary64 (one rounding each for the exponent, pow and the
// division), memoised per host thread for the last theta.
inline void fill_inv_freq(double theta, double* out)
{
    thread_local double last_theta = 0.0;
    thread_local double table[kHeadDim / 2];
    if (theta != last_theta) {
        for (int i = 0; i < kHeadDim / 2; ++i) table[i] = 1.0 / std::pow(theta, (double)(2 * i) / (double)kHeadDim);
        last_theta = theta;
    }
    std::memcpy(out, table, sizeof(table));
}

}  // namespace msa_internal
