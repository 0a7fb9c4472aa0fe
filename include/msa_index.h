/*
 * msa_index.h — C ABI of the MSA indexer (block selection over the index-K cache) for AMD Instinct
 * MI355X (gfx950).  It is the consumer of the index-K cache that msa_produce writes.
 *
 * The operation (page "Fuse MiniMax-M3 MSA per-layer KV-cache writes into one kernel", "Where this PR
 * targets at", step 4: proxy-FMHA over index-K, max-reduce, top-16 of 128-token blocks; page "Fuse
 * MiniMax-M3 QKV and index projection", BEFORE/AFTER figures: score visible index-K, max-pool the
 * scores by block, select the top-k block IDs; page "Wire in custom decode kernels for MinimaxM3",
 * test summary: the top-k table is head-major and per-token valid-block counts are staged):
 *
 *   score(t, h, p)   = scale * sum_d iq[t, h, d] * ik[p, d]   for every key position p visible to t
 *                      (same sequence, 0 <= p <= pos_t, page valid), index-Q head h reading index-K
 *                      head h / (num_iq_heads / num_ik_heads);
 *   block(t, h, b)   = max of score(t, h, p) over the visible p of block b (positions [bB, (b+1)B));
 *   topk(t, h)       = the top_k blocks by block score, descending, equal scores in ascending block
 *                      index, padded with -1.
 *
 * Arithmetic: every product of a bf16 index-Q element and an e4m3 (or bf16) index-K element is exact
 * in binary64, and so is their sum over 128 elements for any realistic range; the score is that sum
 * times the scale (binary64), so the selection does not depend on summation order.  Softmax and the
 * 1/sqrt(head_dim) factor are monotone within one (t, h) and leave the selection unchanged; they are
 * not applied.  A token without a valid cache slot of its own (padded) selects nothing.
 *
 * Conventions are those of msa_produce.h: operands checked for residency on eager calls, no allocation,
 * no synchronisation, all checks on the host before any launch (an error leaves every byte
 * unchanged), MSA_OK means enqueued, graph-capture safe.
 */
#ifndef MSA_INDEX_H
#define MSA_INDEX_H

#include <stdint.h>

#include "msa_produce.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * msa_index_scores — block scores of every (index-Q head, token, block).
 *
 * iq                device bf16 [T, num_iq_heads, head_dim] compact (msa_produce's iq_out), 16-B aligned.
 * num_tokens        T >= 0 (0: nothing launched).
 * head_dim          must be 128.
 * num_iq_heads      >= 1, a multiple of ik_cache->num_heads.
 * positions, seq_idx, page_table, page_table_stride, num_seqs, max_pages_per_seq, page_size,
 * num_pages         the token and page-table metadata msa_produce took (same meaning and checks).
 * ik_cache          host pointer to the index-K cache view (fp8 e4m3 with scale, or bf16).
 * block_tokens      tokens per selection block, > 0 (128 in MiniMax-M3 MSA).
 * max_blocks        row length of block_scores, >= 0; blocks at index >= max_blocks are not scored.
 * block_scores      device double [num_iq_heads, T, max_blocks], 8-B aligned: the block score, or
 *                   -infinity where no key of the block is visible.
 */
msa_status msa_index_scores(const uint16_t* iq, int32_t num_tokens, int32_t head_dim, int32_t num_iq_heads,
                            const int32_t* positions, const int32_t* seq_idx,
                            const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                            int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                            const msa_cache_view* ik_cache, int32_t block_tokens, int32_t max_blocks,
                            double* block_scores, void* stream);

/*
 * msa_index_scores_grouped — msa_index_scores, with keys shared by groups of tokens.  Same arguments
 * and results (every block score bit for bit), plus:
 *
 * group_tokens      1 ..= 8: tokens t = g * group_tokens + i (i < group_tokens) are scored together.
 *                   Tokens of a group that belong to one sequence read each key once for all of
 *                   them, which is what a speculative-decoding verify window (1 + draft_len
 *                   consecutive positions of one sequence, stored next to each other) needs: pass
 *                   its length.  A group whose tokens come from several sequences takes one pass per
 *                   sequence, and padded tokens select nothing, as in msa_index_scores, so any
 *                   grouping gives the same scores; only the speed depends on it.
 *
 * Layouts other than pages and selection blocks of multiples of 64 tokens (blocks of at most 2,048
 * tokens), and group_tokens = 1, run msa_index_scores' kernels.  Errors: those of
 * msa_index_scores; MSA_ERR_SHAPE for group_tokens outside [1, 8].
 */
msa_status msa_index_scores_grouped(const uint16_t* iq, int32_t num_tokens, int32_t head_dim, int32_t num_iq_heads,
                                    const int32_t* positions, const int32_t* seq_idx,
                                    const int32_t* page_table, int64_t page_table_stride, int32_t num_seqs,
                                    int32_t max_pages_per_seq, int32_t page_size, int64_t num_pages,
                                    const msa_cache_view* ik_cache, int32_t block_tokens, int32_t max_blocks,
                                    int32_t group_tokens, double* block_scores, void* stream);

/*
 * msa_index_topk — the top_k blocks of every row of block_scores (as msa_index_scores writes it).
 *
 * block_scores      device double [rows, max_blocks] (rows = num_iq_heads * T), 8-B aligned.
 * rows, max_blocks  >= 0; max_blocks <= 4096.
 * top_k             1 ..= 64.
 * block_ids         device int32 [rows, top_k]: selected block indices, descending score, ties in
 *                   ascending block index, -1 after the last selected block.  Blocks scored
 *                   -infinity or NaN are never selected.
 * counts            optional device int32 [rows]: number of selected blocks.
 */
msa_status msa_index_topk(const double* block_scores, int32_t rows, int32_t max_blocks, int32_t top_k,
                          int32_t* block_ids, int32_t* counts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_INDEX_H */
