/*
 * pa_quest.h - query-aware page selection (Quest) for the paged decode of
 * libpa.so (AMD Instinct MI355X, gfx950).  C ABI; include pa.h first.
 *
 * "KV Cache Engineering for LLM Serving", section 7 (Query-aware sparse
 * reads): the cache is divided into pages; each page keeps the minimum and
 * the maximum of its keys per dimension; a new query scores every page by
 * sum_d max(q_d * min_d, q_d * max_d), the largest q.k any key in the page's
 * box could reach, and attention then reads only the best pages.  Nothing
 * is evicted: all pages stay stored.
 *
 * Here a page is one cache block, and pages are chosen per (sequence, KV
 * head): the query heads of a group share their KV head's K/V, and a page's
 * score for the group is the largest of its query heads' scores.  A decode
 * step is
 *   pa_quest_cache_write(_fp8)   (the write, keeping the summaries current)
 *   pa_quest_select -> pa_decode_quest(_fp8)
 * all on one stream.  Writes with several tokens per block (a prompt) use
 * pa_cache_write(_fp8) followed by pa_quest_update instead.
 *
 * Summaries: a DEVICE array of num_blocks * num_kv_heads * head_dim uint32
 * words, one per (block b, KV head h, dimension d) at index
 *   ((b * (head_dim / 4) + d / 4) * num_kv_heads + h) * 4 + d % 4
 * (for each block and 4 dimensions, the 16-byte quads of all heads are
 * contiguous: the score kernel reads them as one run per page).  A word is
 * (max << 16) | min, both bf16 bit patterns of the keys' stored values (bf16
 * keys as stored; fp8 keys as their e4m3 code values without the per-tensor
 * scale - a positive scale changes no minimum, maximum or ranking).  An
 * empty summary is min = +inf, max = -inf.  NaN keys are ignored.  Start a
 * pool with pa_quest_clear.
 */
#ifndef PA_QUEST_H_
#define PA_QUEST_H_

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Sets every summary word of the pool empty (a fill kernel on `stream`).
 * summaries: DEVICE, num_blocks * num_kv_heads * head_dim uint32.           */
pa_status pa_quest_clear(const pa_cache_desc* cache, uint32_t* summaries, void* stream);

/* pa_cache_write in one launch with the summary update: the caches are
 * written exactly as pa_cache_write writes them, and the summaries end as
 * pa_cache_write followed by pa_quest_update leaves them (a token at offset
 * 0 starts its block's summary afresh, every token widens its block's).
 * Contract: no two tokens of one call go to the same block - a decode
 * step's new tokens, one per sequence, each appended to a block that its
 * sequence alone holds (copy-on-write guarantees that).  Several tokens in
 * one block give undefined summaries (the caches are still written as
 * pa_cache_write writes them).
 *   summaries  DEVICE, as for pa_quest_update; NULL -> PA_ERR_NULL (unless
 *              num_tokens == 0)
 * Other arguments and errors as pa_cache_write.                            */
pa_status pa_quest_cache_write(const pa_cache_desc* cache, const void* k, const void* v,
                               const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                               void* v_cache, uint32_t* summaries, void* stream);

/* The same into an fp8 (e4m3fn) cache, as pa_cache_write_fp8: the summaries
 * take the stored codes' values.                                             */
pa_status pa_quest_cache_write_fp8(const pa_cache_desc* cache, const void* k, const void* v,
                                   const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                                   void* v_cache, float k_scale, float v_scale, uint32_t* summaries,
                                   void* stream);

/* Keeps the summaries current after a cache write of the same tokens
 * (call it after pa_cache_write / pa_cache_write_fp8 on the same stream):
 * every block that received a token at offset 0 starts empty, then each
 * written token's stored key (read back from k_cache) widens its block's
 * words.  Slots that are negative or outside the pool are skipped, as the
 * write skips them.  This keeps a block's summary equal to the min/max of
 * the tokens written to it since its first token, as long as every write to
 * the block goes through this call; a block filled another way (a block
 * copy, a swap-in) needs pa_quest_summarize.
 *   elem_bytes    2 (bf16 cache) or 1 (fp8 cache)
 *   slot_mapping  DEVICE [num_tokens] int64, as given to the cache write    */
pa_status pa_quest_update(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, uint32_t* summaries,
                          void* stream);

/* Recomputes the summaries of blocks[i] (DEVICE int32, i < num_items) from
 * their first counts[i] tokens (DEVICE int32, clamped to [0, block_size]).
 * Ids outside the pool are skipped.                                          */
pa_status pa_quest_summarize(const pa_cache_desc* cache, int32_t elem_bytes, const void* k_cache,
                             const int32_t* blocks, const int32_t* counts, int32_t num_items,
                             uint32_t* summaries, void* stream);

/* Bytes of DEVICE workspace pa_quest_select needs (page score keys); 0 for
 * invalid sizes.                                                             */
size_t pa_quest_select_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                      int32_t max_blocks_per_seq);

/* Chooses, for each (sequence s, KV head h), the `budget` pages of s with
 * the highest scores for the query heads h*G .. h*G+G-1 (G = num_q_heads /
 * num_kv_heads; G <= 16):
 *   score(page) = max over those heads of  sum_{d = 0..D-1} max(q_d * min_d, q_d * max_d)
 * with float32 products and a float32 sum taken in dimension order (the
 * order is part of the definition: it decides which pages are read; the
 * products of bf16 values are exact unless below 2^-134 in magnitude, and
 * the kernel adds each as a fused multiply-add).  Each page's summary must
 * be non-empty (a page below L holds a written or summarized token).  Equal
 * scores go to the lower page index.  The chosen pages' block ids are
 * written in page order to sel_tables[s * Hkv + h][0 .. budget), and
 * sel_lens[s * Hkv + h] gets the tokens they hold (budget * block_size, less
 * the empty tail of the sequence's last page when it is chosen).  A
 * sequence with at most `budget` pages keeps all of them (its table row is
 * copied, entries past its pages set to -1, and sel_lens = L): that is
 * plain decode.  A length outside [0, max_blocks * block_size] gives
 * sel_lens = -1, which pa_decode_quest turns into NaN rows.
 *   q             DEVICE [num_seqs][num_q_heads][head_dim] bf16
 *   summaries     DEVICE, as kept by pa_quest_update / pa_quest_summarize
 *   block_tables  DEVICE [num_seqs][max_blocks_per_seq] int32
 *   seq_lens      DEVICE [num_seqs] int32
 *   budget        >= 1 pages per (sequence, KV head)
 *   sel_tables    DEVICE [num_seqs * num_kv_heads][budget] int32 (output)
 *   sel_lens      DEVICE [num_seqs * num_kv_heads] int32 (output)
 *   workspace     DEVICE, >= pa_quest_select_workspace_size bytes, any contents
 * PA_ERR_SHAPE / PA_ERR_UNSUPPORTED / PA_ERR_WORKSPACE on bad arguments.    */
pa_status pa_quest_select(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                          int32_t num_q_heads, const uint32_t* summaries,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* seq_lens, int32_t budget, int32_t* sel_tables,
                          int32_t* sel_lens, void* workspace, size_t workspace_bytes, void* stream);

/* Decode workspace for pa_decode_quest(_fp8): zero-filled once, and reused
 * under pa_decode's rule, with one merge counter per (sequence, KV head), so
 * U = num_seqs * num_kv_heads.  0 for invalid sizes.                        */
size_t pa_decode_quest_workspace_size(const pa_cache_desc* cache, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t budget,
                                      int32_t partition_tokens);

/* Paged decode over the chosen pages: out[s, i, :] is softmax attention of
 * query head i over the tokens of sel_tables[s * Hkv + h] (h = i / G, the
 * first sel_lens[s * Hkv + h] of them), exactly as pa_decode computes it
 * over a full block table.  Arguments as pa_decode, with the selection in
 * place of block_tables / max_blocks_per_seq / seq_lens.                   */
pa_status pa_decode_quest(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                          int32_t num_q_heads, const void* k_cache, const void* v_cache,
                          const int32_t* sel_tables, int32_t budget, const int32_t* sel_lens,
                          float scale, float* out, int32_t partition_tokens, void* workspace,
                          size_t workspace_bytes, void* stream);

/* The same over an fp8 (e4m3fn) cache, with pa_decode_fp8's scales.        */
pa_status pa_decode_quest_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                              int32_t num_q_heads, const void* k_cache, const void* v_cache,
                              const int32_t* sel_tables, int32_t budget, const int32_t* sel_lens,
                              float scale, float k_scale, float v_scale, float* out,
                              int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_QUEST_H_ */
