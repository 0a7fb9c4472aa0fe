/*
 * msa_unfused.h — C ABI of the unfused producer path for AMD Instinct MI355X (gfx950): the same
 * outputs as msa_produce (bit for bit), computed the way the write path ran before it was fused.
 *
 * The structure it reproduces (page "Fuse MiniMax-M3 MSA per-layer KV-cache writes into one
 * kernel", "The problem": each of the three cache writes, K, V and index-K, takes four small
 * kernels, a division, a remainder, an index cast and an indexed scatter, so twelve per sparse
 * layer; page "Fuse MiniMax-M3 QKV and index projection", BEFORE figure: a main producer applies
 * Q/K norm and RoPE and an index producer does the same for index-Q/index-K).  One call runs
 *
 *   main producer    Q, K heads: RMSNorm + RoPE; Q to q_out (bf16), K to a binary32 workspace;
 *   index producer   index-Q, index-K heads likewise (index-Q to iq_out, index-K to the workspace);
 *   per cache (K, V, index-K), four launches:
 *     division       page   = slot / page_size            (-1 for a slot < 0)
 *     remainder      offset = slot % page_size             (-1 for a slot < 0)
 *     index cast     element index of (page, head 0, offset, 0) in 64 bits, or -1 when the
 *                    slot is < 0 or its page is outside [0, num_pages)
 *     scatter        cast and store each head row at that index (V from the raw input row)
 *
 * i.e. 14 launches for a layer with all five streams against msa_produce's one.  Every value is
 * rounded exactly as msa_produce rounds it (the normalised K and index-K pass through binary32,
 * which holds them exactly), so the two paths write identical bytes.
 *
 * The pages keep the per-cache path for cache layouts the fused kernel does not take ("Fuse
 * MiniMax-M3 MSA per-layer KV-cache writes into one kernel", summary).  Here that means: the
 * unfused scatter accepts any positive, non-overlapping cache strides and a data pointer aligned
 * to its element size, where msa_produce requires strides in multiples of 8 elements and a 16-byte
 * aligned base (MSA_ERR_STRIDE / MSA_ERR_ALIGNMENT there).
 *
 * Conventions are those of msa_produce.h: operands checked for residency on eager calls, no allocation
 * (intermediates live in the caller's workspace), no synchronisation, every check on the host
 * before any launch (an error leaves every byte unchanged), MSA_OK means enqueued, graph-capture
 * safe.
 */
#ifndef MSA_UNFUSED_H
#define MSA_UNFUSED_H

#include <stddef.h>
#include <stdint.h>

#include "msa_produce.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * msa_slots — the cache slot of every token, one launch (the step-level metadata the unfused
 * path takes as input; page "Wire in custom decode kernels for MinimaxM3", commit notes: slots
 * derived from the page table).
 *
 * positions, seq_idx, page_table, page_table_stride, num_seqs, max_pages_per_seq, page_size,
 * num_pages   as in msa_produce, with the same validity rule.
 * slots_out   device int64 [T], 8-byte aligned: page * page_size + position % page_size, or -1.
 */
msa_status msa_slots(const int32_t* positions, const int32_t* seq_idx, int32_t num_tokens,
                     const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                     int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                     int64_t* slots_out, void* stream);

/*
 * msa_produce_unfused_workspace_size — bytes of workspace msa_produce_unfused needs for T tokens:
 * binary32 K and index-K rows plus three (page, offset, index) int64 arrays per cache, each
 * region 256-byte aligned.  MSA_ERR_SHAPE for negative counts.
 */
msa_status msa_produce_unfused_workspace_size(int32_t num_tokens, int32_t num_kv_heads, int32_t num_ik_heads,
                                              uint64_t* bytes);

/*
 * msa_produce_unfused — one layer through the unfused path (see above).
 *
 * x, x_row_stride, num_tokens, head_dim, num_*_heads, positions, *_norm_weight, rms_eps,
 * rope_theta, q_out, iq_out   as in msa_produce (same requirements).
 * slots           device int64 [T] (msa_slots, or msa_produce's slots_out): slot of each token,
 *                 < 0 for none.  A slot whose page is outside [0, num_pages) is skipped; valid
 *                 slots must be distinct.
 * page_size       > 0; num_pages >= 0.
 * k_cache, v_cache, ik_cache   cache descriptors as in msa_produce, except that any positive,
 *                 non-overlapping strides are accepted and `data` need only be aligned to its
 *                 element size.
 * workspace       device memory of at least msa_produce_unfused_workspace_size bytes, 256-byte
 *                 aligned (MSA_ERR_WORKSPACE otherwise); its contents on entry do not matter
 *                 and it must not be reused by another call until this one has run.
 */
msa_status msa_produce_unfused(const uint16_t* x, int64_t x_row_stride, int32_t num_tokens, int32_t head_dim,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t num_iq_heads,
                               int32_t num_ik_heads, const int32_t* positions, const int64_t* slots,
                               int32_t page_size, int64_t num_pages,
                               const uint16_t* q_norm_weight, const uint16_t* k_norm_weight,
                               const uint16_t* iq_norm_weight, const uint16_t* ik_norm_weight,
                               float rms_eps, double rope_theta,
                               uint16_t* q_out, uint16_t* iq_out,
                               const msa_cache_view* k_cache, const msa_cache_view* v_cache,
                               const msa_cache_view* ik_cache,
                               void* workspace, uint64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_UNFUSED_H */
