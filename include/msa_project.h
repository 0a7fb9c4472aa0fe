/*
 * msa_project.h — C ABI of the packed projection for AMD Instinct MI355X (gfx950), alone and with
 * the producer fused into its epilogue.
 *
 * The projection (page "Fuse MiniMax-M3 QKV and index projection", AFTER figure: one wider GEMM of
 * the hidden states produces the packed row [Q | K | V | index-Q | index-K]):
 *
 *   x[t, c] = bf16( sum_k h[t, k] * w[c, k] )
 *
 * h: bf16 hidden states [T, K]; w: bf16 packed weight [N, K] (one row per output column, the
 * layout of a linear layer's weight); x: bf16 [T, N].  The sum runs on the matrix cores (bf16
 * products, binary32 accumulation) in an order fixed by the kernel: the same inputs always give
 * the same bits, but not the bits of an exact sum.  For any accumulation order the binary32 sum
 * lies within K * 2^-24 / (1 - K * 2^-24) * sum_k |h[t, k] w[c, k]| of the exact one, before the
 * final rounding to bf16.
 *
 * msa_project_produce runs the same GEMM (same kernel, same accumulation order) and, instead of
 * storing x, hands each head's bf16-rounded row to the producer's arithmetic (msa_produce.h):
 * per-head RMSNorm + neox RoPE on Q, K, index-Q and index-K, compact Q and index-Q, and K, V,
 * index-K into the paged caches.  Its outputs equal msa_produce applied to msa_project's x: bit for
 * bit up to 1,024 tokens (the same operations in the same order), and for larger batches except
 * where a head's binary64 sum of squares is inexact (a head spanning more than about 2^15 in
 * magnitude), where the two sum orders may differ in the last binary64 bit.  The packed row never
 * touches memory.  The pages stop at a single wider GEMM feeding a separate fused producer; this
 * entry point goes one step further.
 *
 * Kernels: for up to 1,024 tokens (the decode and verify batches) one split-K launch (heads x
 * 64-token chunks x K slices, on v_mfma_f32_32x32x16_bf16): the slices of a head and chunk leave
 * their partial sums in the workspace, then each adds one group of 8 tokens over all slices in a
 * fixed order and runs the epilogue in msa_produce's row layout; for larger batches (prefill) one
 * 256 x 256 tiled kernel on the same matrix instruction.
 *
 * Conventions are those of msa_produce.h (operands checked for residency on eager calls, no allocation,
 * no synchronisation, all checks on the host before any launch, MSA_OK means enqueued,
 * graph-capture safe).
 */
#ifndef MSA_PROJECT_H
#define MSA_PROJECT_H

#include <stdint.h>

#include "msa_produce.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * msa_project_workspace_size — bytes of workspace (device memory, 256-byte aligned) a projection of
 * num_tokens rows of width hidden onto num_heads heads of 128 columns needs (both entry points
 * take the same).  Zero for batches above 1,024 tokens (one tiled kernel, no workspace).  Up to
 * 1,024 tokens the projection is one split-K launch whose work-groups exchange partial sums in the
 * workspace: a 256-byte header (uint32 word 1: an error word), then the partial sums, each stored
 * as the bitwise complement of its binary32 bits so that a zero word means "not written yet".
 * Every partial sum is read once and cleared by the work-group that reads it.
 *
 * The workspace must be zero-filled before its first use; every call that completes leaves it all
 * zero again, so no call needs it cleared, whatever its sizes.  Calls that share a workspace must
 * not overlap in time (same stream, or ordered).  A work-group waits (polls) only for the other K
 * slices of its own head and 64-token chunk, a bounded number of times: if a call starts on a
 * workspace that is not all zero, its outputs may be wrong and the workspace is left dirty, and if
 * a wait gives up (the device cannot hold one head's slices at once, at most 63 work-groups), the
 * call sets error bits in the error word and leaves that token group's outputs unwritten.  No
 * state of the workspace can make a call hang.  The error word is only ever set, never cleared,
 * by the library.
 *
 * SHAPE when hidden is not a positive multiple of 64, num_heads is outside [1, 4096], or (1 to
 * 1,024 tokens) hidden exceeds 24,192 = 63 x 384 (at most 63 K slices per head and chunk).
 */
msa_status msa_project_workspace_size(int32_t num_tokens, int32_t hidden, int32_t num_heads, uint64_t* bytes);

/*
 * msa_project — the packed projection alone.
 *
 * h            device bf16 [T, hidden], row stride h_row_stride (>= hidden, multiple of 8), 16-B aligned.
 * num_tokens   T >= 0 (0: nothing launched).
 * hidden       K: a positive multiple of 64.
 * w            device bf16 [num_cols, hidden], row stride w_row_stride (>= hidden, multiple of 8), 16-B aligned.
 * num_cols     N: a positive multiple of 128, at most 4096 * 128.
 * x_out        device bf16 [T, num_cols], row stride x_row_stride (>= num_cols, multiple of 8), 16-B aligned.
 * workspace    as msa_project_workspace_size states; may be NULL when it gives 0.
 *
 * STRIDE also when T > 1,024 and h_row_stride or w_row_stride is 2^22 elements or more (the tiled
 * kernel addresses a tile's 256 rows with 32-bit offsets).
 */
msa_status msa_project(const uint16_t* h, int64_t h_row_stride, int32_t num_tokens, int32_t hidden,
                       const uint16_t* w, int64_t w_row_stride, int32_t num_cols,
                       uint16_t* x_out, int64_t x_row_stride,
                       void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * msa_project_produce — the projection with the producer as its epilogue.
 *
 * h, h_row_stride, num_tokens, hidden, w, w_row_stride   as in msa_project; w has
 *              (num_q_heads + 2 num_kv_heads + num_iq_heads + num_ik_heads) * head_dim rows in the
 *              packed order Q, K, V, index-Q, index-K.
 * head_dim, num_*_heads, *_norm_weight, rms_eps, q_out, iq_out, k_cache, v_cache, ik_cache
 *              as in msa_produce (same requirements).
 * rope_cos, rope_sin   device float [T, head_dim / 2], 16-B aligned: the RoPE coefficients of each
 *              token, as msa_rope_table computes them from the positions (once per step; every
 *              layer of the step reads the same table).
 * slots        device int64 [T], 8-B aligned: the cache slot of each token (msa_slots, or
 *              msa_produce's slots_out); < 0, or a page outside [0, num_pages): no cache write.
 *              Valid slots must be distinct.
 * page_size    > 0; num_pages >= 0.
 * workspace    as msa_project_workspace_size states.
 */
msa_status msa_project_produce(const uint16_t* h, int64_t h_row_stride, int32_t num_tokens, int32_t hidden,
                               const uint16_t* w, int64_t w_row_stride, int32_t head_dim,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads,
                               int32_t num_ik_heads, const float* rope_cos, const float* rope_sin,
                               const int64_t* slots, int32_t page_size, int64_t num_pages,
                               const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                               const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                               float rms_eps, uint16_t* q_out, uint16_t* iq_out,
                               const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                               const msa_cache_view* ik_cache,
                               void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * msa_project_produce_noalloc — msa_project_produce without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It allocates nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 * The split-K partial sums go to a scratch array the library owns: 32 MiB (33,554,432 bytes) of
 * device memory per GPU, part of the library's code object, held by every GPU the library runs on
 * until the process ends.  A call whose workspace need (msa_project_workspace_size) exceeds it
 * returns MSA_ERR_WORKSPACE before touching the device: 23 heads of hidden 3,072 fit up to 256
 * tokens; batches above 1,024 tokens need no scratch and always fit.  The first call on a device
 * looks up that device's copy of the array (a runtime query that allocates nothing); if the runtime
 * refuses such queries during graph capture, make one eager call first.
 *
 * Every call on one GPU shares that GPU's array.  It starts zeroed, as a workspace must, and each
 * completed call leaves it all zero again.  Calls that overlap in time on one GPU (different
 * streams without ordering between them, or several host threads) race on it, give wrong results
 * and may leave it dirty for later calls; calls on one stream, or otherwise ordered, are safe.
 *
 * Arguments, results and the other errors: as msa_project_produce, minus workspace and
 * workspace_bytes.
 */
msa_status msa_project_produce_noalloc(const uint16_t* h, int64_t h_row_stride, int32_t num_tokens, int32_t hidden,
                                       const uint16_t* w, int64_t w_row_stride, int32_t head_dim,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads,
                                       int32_t num_ik_heads, const float* rope_cos, const float* rope_sin,
                                       const int64_t* slots, int32_t page_size, int64_t num_pages,
                                       const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                                       const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                                       float rms_eps, uint16_t* q_out, uint16_t* iq_out,
                                       const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                                       const msa_cache_view* ik_cache, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PROJECT_H */
