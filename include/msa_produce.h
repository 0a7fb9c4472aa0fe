/*
 * msa_produce.h — C ABI of the MiniMax-M3 MSA fused producer for AMD Instinct MI355X (gfx950).
 *
 * The operation (pages "Fuse MiniMax-M3 QKV and index projection", AFTER figure and change
 * list, and "Fuse MiniMax-M3 MSA per-layer KV-cache writes into one kernel", sections "The
 * problem" / "The fix" / "Nsys trace"): for every new token, read one row of the packed
 * projection output [Q | K | V | index-Q | index-K]; apply per-head RMSNorm and neox RoPE to the
 * Q, K, index-Q and index-K heads; emit compact bf16 Q and index-Q; compute the token's cache
 * page and in-page offset once from the page table; write K, V and index-K into paged HND
 * caches (OCP FP8 E4M3 or bf16), skipping padded and out-of-range slots.  Write slots come from
 * the per-request page table (page "Wire in custom decode kernels for MinimaxM3", notes of the
 * conflict-resolution commit), not from a per-token slot buffer.
 *
 * Arithmetic (the pages fix no precision; this is the reading implemented and tested):
 *   inv_freq_i = 1 / theta^(2i/D), angle = pos * inv_freq_i (binary64);
 *   c_i = (float)cos(angle), s_i = (float)sin(angle);
 *   r = (float)(1 / sqrt(sum_j a_j^2 / D + eps)) with the sum and the rest in binary64;
 *   y_j = (a_j * r) * w_j, o_i = y_i c_i - y_{i+D/2} s_i, o_{i+D/2} = y_{i+D/2} c_i + y_i s_i
 *   (binary32, one rounding per operation, no fused multiply-add);
 *   Q/index-Q = bf16_rne(o); cache: fp8 = e4m3_rne_satfinite(v * (float)(1/scale)),
 *   bf16 = bf16_rne(v), where v = o for K and index-K and v = a (the raw input) for V.
 *   NaN inputs give NaN outputs of the same sign.
 *
 * Conventions of every entry point:
 *   - Pointers marked "device" must be memory that kernels on the current HIP device can access:
 *     device memory of that device, managed memory, or pinned host memory mapped at the same
 *     address.  An eager call (its stream not being captured into a graph) checks this for every
 *     operand before launching, together with the operand's extent (the bytes the call may touch
 *     must lie inside the allocation the runtime reports), and returns MSA_ERR_NOT_DEVICE without
 *     launching when a check fails (msa_check_device_pointers runs the same check alone).  While the
 *     stream is being captured the check is skipped: the caller keeps captured operands valid for
 *     every replay.  The library allocates nothing, keeps no pointer after it returns, performs no
 *     host<->device copy and no synchronisation, so every call may be captured into a HIP graph.
 *   - `stream` is a hipStream_t (NULL = the null stream).  MSA_OK means the work was enqueued;
 *     device-side faults surface at the caller's next synchronisation.
 *   - Every argument check runs on the host before any launch: on any status other than MSA_OK
 *     nothing was launched and no output byte changed.
 *   - The only state the library keeps between calls is a per-host-thread memo of the RoPE
 *     inverse frequencies for the last theta (a pure function of theta); concurrent calls from
 *     several host threads are safe as long as their outputs do not overlap.
 */
#ifndef MSA_PRODUCE_H
#define MSA_PRODUCE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msa_status {
    MSA_OK = 0,
    MSA_ERR_NULL_POINTER = 1,   /* a required pointer is NULL */
    MSA_ERR_UNSUPPORTED = 2,    /* head_dim other than 128 */
    MSA_ERR_SHAPE = 3,          /* negative count, no heads, table/cache geometry mismatch */
    MSA_ERR_STRIDE = 4,         /* stride too small, overlapping cache rows, or not a multiple of 8 elements */
    MSA_ERR_ALIGNMENT = 5,      /* a pointer not aligned as documented */
    MSA_ERR_DTYPE = 6,          /* unknown cache dtype, or an fp8 cache without a scale */
    MSA_ERR_OVERFLOW = 7,       /* a cache element offset does not fit in int64 */
    MSA_ERR_LAUNCH = 8,         /* the HIP runtime refused the launch */
    MSA_ERR_WORKSPACE = 9,      /* a caller-provided workspace is too small or misaligned */
    MSA_ERR_NOT_DEVICE = 10     /* an operand is not accessible from the current device, or the bytes
                                   the call would touch run past the end of its allocation */
} msa_status;

typedef enum msa_cache_dtype {
    MSA_CACHE_FP8_E4M3 = 0,     /* OCP FP8 E4M3 ("E4M3FN"), 1 byte per element */
    MSA_CACHE_BF16 = 1          /* bfloat16, 2 bytes per element */
} msa_cache_dtype;

/*
 * One paged HND cache: logical shape [num_pages, num_heads, page_size, head_dim] (pages
 * "Fuse MiniMax-M3 QKV and index projection", change list: paged HND cache storage, strided
 * layouts allowed).  Element (page, head, token, d) is at element offset
 *     page * stride_page + head * stride_head + token * stride_token + d
 * from `data` (the dim stride is 1).  Offsets are computed in 64-bit arithmetic.
 * Requirements: data 16-byte aligned; every stride a positive multiple of 8 elements; the view
 * must not overlap itself (sorted by stride, each stride >= the previous stride times its
 * extent); the largest offset must fit in int64.  The caller owns the memory; cache bytes of
 * tokens without a valid slot, and every byte outside the view, are never written.
 */
typedef struct msa_cache_view {
    void* data;                 /* device */
    int64_t stride_page;        /* elements */
    int64_t stride_head;        /* elements */
    int64_t stride_token;       /* elements */
    int32_t num_heads;          /* must equal num_kv_heads (K, V) or num_ik_heads (index-K) */
    int32_t dtype;              /* msa_cache_dtype */
    const float* scale;         /* device fp32[1]: per-tensor dequantisation scale (stored = value / scale);
                                   required for FP8, ignored for BF16.  Read at run time, so a captured
                                   graph picks up a new scale without recapture. */
} msa_cache_view;

/*
 * msa_produce — the fused producer for one layer and one batch of tokens (one launch).
 *
 * x                  device bf16, row t at x + t * x_row_stride (elements); the first
 *                    W = (num_q_heads + 2*num_kv_heads + num_iq_heads + num_ik_heads) * head_dim
 *                    columns hold Q heads, then K, V, index-Q, index-K heads, head_dim each
 *                    (page "Fuse MiniMax-M3 QKV and index projection", AFTER figure).
 *                    16-byte aligned; x_row_stride >= W and a multiple of 8.
 * num_tokens         T >= 0.  T == 0 returns MSA_OK without launching.
 * head_dim           must be 128.
 * num_*_heads        local heads of one tensor-parallel rank; num_kv_heads >= 1 or any other
 *                    count >= 1 (at least one head in total); each >= 0.
 * positions          device int32 [T]: token position within its sequence (RoPE angle and slot).
 * seq_idx            device int32 [T]: row of page_table; a value < 0 marks a padded token.
 * page_table         device int32 [num_seqs, page_table_stride]: physical page of each logical
 *                    page (logical page = position / page_size).  May be NULL when num_seqs == 0.
 * page_table_stride  elements between rows, >= max_pages_per_seq.
 * num_seqs, max_pages_per_seq, page_size (> 0), num_pages (>= 0): table and pool geometry.
 *                    A token writes its cache slot only if 0 <= seq < num_seqs, position >= 0,
 *                    position / page_size < max_pages_per_seq and 0 <= page < num_pages
 *                    (page "Fuse MiniMax-M3 QKV and index projection", change list: padded or
 *                    out-of-range cache slots are contained).  Invalid slots are not errors.
 *                    Valid slots must be distinct within one call (not checked on the device).
 * *_norm_weight      device bf16 [head_dim] per stream, shared by that stream's heads, 16-byte
 *                    aligned; NULL allowed when the stream has no heads.
 * rms_eps            RMSNorm epsilon (>= 0).
 * rope_theta         RoPE base (> 0).
 * q_out              device bf16 [T, num_q_heads, head_dim] compact, 16-byte aligned.
 * iq_out             device bf16 [T, num_iq_heads, head_dim] compact, 16-byte aligned.
 *                    Q and index-Q rows are written for every token, padded ones included.
 * k_cache, v_cache   host pointers to cache descriptors (num_heads == num_kv_heads);
 * ik_cache           (num_heads == num_ik_heads).  A descriptor may be NULL when its head count is 0.
 * slots_out          optional device int64 [T], 8-byte aligned: slot = page * page_size + offset,
 *                    or -1 when the token wrote nothing.
 * stream             hipStream_t.
 */
msa_status msa_produce(const uint16_t* x, int64_t x_row_stride, int32_t num_tokens, int32_t head_dim,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads, int32_t num_ik_heads,
                       const int32_t* positions, const int32_t* seq_idx,
                       const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                       int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                       const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                       const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                       float rms_eps, double rope_theta,
                       uint16_t* q_out, uint16_t* iq_out,
                       const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                       const msa_cache_view* ik_cache,
                       int64_t* slots_out, void* stream);

/*
 * msa_rope_table — the RoPE coefficients msa_produce uses, alone (same device code):
 * cos_out[t, i] = (float)cos(positions[t] * inv_freq_i), sin_out likewise, i < head_dim / 2.
 * positions device int32 [n]; cos_out, sin_out device float [n, head_dim / 2].
 * head_dim must be 128; rope_theta > 0; n >= 0.
 */
msa_status msa_rope_table(const int32_t* positions, int64_t n, double rope_theta, int32_t head_dim,
                          float* cos_out, float* sin_out, void* stream);

/*
 * msa_quantize — the output casts msa_produce uses, alone (same device code).
 * dtype MSA_CACHE_FP8_E4M3: codes_out uint8 [n] = e4m3_rne_satfinite(values * (float)(1 / *scale));
 * dtype MSA_CACHE_BF16:     codes_out uint16 [n] = bf16_rne(values) (scale ignored, may be NULL).
 * values device float [n]; scale device float[1]; codes_out device, n >= 0.
 */
msa_status msa_quantize(const float* values, int64_t n, int32_t dtype, const float* scale, void* codes_out,
                        void* stream);

/*
 * msa_rms_scale — the RMSNorm scale msa_produce uses, alone (same device code):
 * r_out[i] = (float)(1 / sqrt(sum_sq[i] / head_dim + rms_eps)) in binary64.
 * sum_sq device double [n]; r_out device float [n]; head_dim must be 128.
 */
msa_status msa_rms_scale(const double* sum_sq, int64_t n, int32_t head_dim, float rms_eps, float* r_out,
                         void* stream);

/*
 * msa_check_device_pointers — the operand check of eager calls, alone (launches nothing).
 *
 * ptrs     host array [n] of pointers; NULL entries pass.
 * bytes    host array [n]: bytes from ptrs[i] that a kernel may touch (NULL: one byte each).
 * n        >= 0.
 * first_bad optional: the index of the first pointer that fails, or -1.
 * Returns MSA_OK when every pointer is accessible from the current device with its whole extent
 * inside its allocation, MSA_ERR_NOT_DEVICE otherwise (also when no device is present), and
 * MSA_ERR_NULL_POINTER / MSA_ERR_SHAPE for a NULL ptrs array with n > 0 / n < 0.
 */
msa_status msa_check_device_pointers(const void* const* ptrs, const uint64_t* bytes, int32_t n, int32_t* first_bad);

/* Static English text for a status code. */
const char* msa_status_string(msa_status status);

/* The same text under the shorter name. */
const char* msa_status_str(msa_status status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PRODUCE_H */
