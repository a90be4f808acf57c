/*
 * pa_cascade.h - shared-prefix (cascade) decode for libpa.so (AMD Instinct
 * MI355X, gfx950).  C ABI; include pa.h first.
 *
 * Sequences whose prompts start alike hold the same physical blocks for that
 * prefix ("Taming the token torrent", "Implementing Radix Tree Prefix
 * Caching"; "KV Cache Engineering for LLM Serving", section 11).  Softmax
 * attention splits at any token into parts whose partial states merge
 * exactly by log-sum-exp, so the shared blocks can be attended to once for
 * all the sequences that hold them, and each sequence's own blocks by the
 * ordinary paged decode.  The result is pa_decode's, within the same
 * tolerances; only the order of the sums differs.
 *
 * A step is:
 *   host:   pa_cascade_plan_build from the batch's block tables (host arrays,
 *           as pa_bm_batch returns them), then pa_cascade_plan_export into
 *           host arrays, copied to the device;
 *   device: pa_decode_cascade(_fp8) with those arrays.
 * A plan depends only on the tables and lengths; it is rebuilt when they
 * change.
 *
 * Segments: two sequences share logical block j when their tables agree on
 * blocks 0..j and block j is full for both.  A segment is a maximal run of
 * blocks shared by one and the same set of at least two sequences.  Each
 * sequence's private part is the rest of its tokens, after its last shared
 * block (a partly filled last block is always private).
 */
#ifndef PA_CASCADE_H_
#define PA_CASCADE_H_

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_cascade_plan pa_cascade_plan;

/* Wavefronts per workgroup of the shared-segment kernel; a workgroup takes
 * PA_CASCADE_WAVES * (16 / G) member sequences of a segment chunk.          */
#define PA_CASCADE_WAVES 8

/* Most blocks one workgroup of the shared-segment kernel takes: the segment
 * chunk's block ids are held in on-chip memory.                              */
#define PA_CASCADE_MAX_CHUNK_BLOCKS 256

typedef struct {
  int32_t num_segments;
  int32_t num_items;              /* workgroups of the shared part */
  int32_t num_slots;              /* partial records: one per (segment chunk, member) */
  int32_t num_seg_blocks;
  int32_t num_members;            /* sum over segments of their members */
  int32_t num_parts;              /* sum over sequences of their partial records */
  int32_t members_per_workgroup;  /* PA_CASCADE_WAVES * (16 / G) */
  int32_t chunk_blocks;           /* blocks per segment chunk */
  int64_t shared_tokens;          /* sum over segments of tokens x members: per-sequence reads replaced */
  int64_t segment_tokens;         /* sum over segments of tokens: what is read once instead */
} pa_cascade_plan_info;

/* Builds the plan of a batch.  HOST inputs: block_tables [num_seqs]
 * [max_blocks_per_seq] int32, seq_lens [num_seqs] int32.  chunk_tokens (>= 1)
 * sets how many tokens of a segment one workgroup takes (rounded down to
 * whole blocks, at least one and at most PA_CASCADE_MAX_CHUNK_BLOCKS).  Lengths outside [0, max_blocks * block_size]
 * share nothing and keep their length (the decode turns them into NaN rows).
 * PA_ERR_SHAPE for bad sizes, PA_ERR_UNSUPPORTED for G = num_q_heads /
 * num_kv_heads > 16.                                                        */
pa_status pa_cascade_plan_build(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t block_size, int32_t num_kv_heads,
                                int32_t num_q_heads, int32_t chunk_tokens, pa_cascade_plan** out);

/* Frees a plan; NULL is a no-op.                                             */
void pa_cascade_plan_destroy(pa_cascade_plan* plan);

/* Sizes of the arrays pa_cascade_plan_export writes.                         */
pa_status pa_cascade_plan_get_info(const pa_cascade_plan* plan, pa_cascade_plan_info* info);

/* Copies the plan into HOST arrays (sizes from the info):
 *   items           [num_items][8] int32
 *   seg_blocks      [num_seg_blocks]
 *   members         [num_members]
 *   parts_off       [num_seqs + 1]
 *   parts           [num_parts]
 *   private_tables  [num_seqs][max_blocks_per_seq] (entries past a sequence's
 *                   private blocks are -1)
 *   private_lens    [num_seqs]
 *   segments        [num_segments][4] {first block, blocks, members offset,
 *                   members}: for inspection only; may be NULL
 * The others must not be NULL unless their size is 0.                       */
pa_status pa_cascade_plan_export(const pa_cascade_plan* plan, int32_t* items, int32_t* seg_blocks,
                                 int32_t* members, int32_t* parts_off, int32_t* parts,
                                 int32_t* private_tables, int32_t* private_lens, int32_t* segments);

/* The exported arrays, on the DEVICE.                                        */
typedef struct {
  const int32_t* items;
  int32_t num_items;
  const int32_t* seg_blocks;
  const int32_t* members;
  const int32_t* parts_off;
  const int32_t* parts;
  int32_t num_slots;
  const int32_t* private_tables;
  const int32_t* private_lens;
} pa_cascade_device_plan;

/* DEVICE workspace bytes of pa_decode_cascade(_fp8): the private decode's
 * workspace first (its merge counters in the first max(U, 16384) * 4 + 65,536 bytes,
 * U = num_seqs * num_kv_heads), then the private outputs and the partial
 * records, which each call writes before reading.  Zero-fill it once (as
 * pa_decode's); it then serves any number of calls with any plan and sizes
 * that fit while U <= 16384, exactly as pa_decode's workspace does.  0 for
 * invalid sizes.                                                             */
size_t pa_decode_cascade_workspace_size(const pa_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
                                        int32_t max_blocks_per_seq, int32_t num_slots,
                                        int32_t partition_tokens);

/* Decode of the batch the plan was built from: out[s, i, :] as pa_decode
 * computes it (q, caches, scale, out, partition_tokens as there;
 * max_blocks_per_seq is the tables' width the plan was built with).  Three
 * kernels on `stream`: the shared segments, the private parts (the paged
 * decode over private_tables / private_lens, which also returns each row's
 * log-sum-exp), and the merge.                                               */
pa_status pa_decode_cascade(const pa_cache_desc* cache, const void* q, int32_t num_seqs, int32_t num_q_heads,
                            const void* k_cache, const void* v_cache, int32_t max_blocks_per_seq,
                            const pa_cascade_device_plan* plan, float scale, float* out,
                            int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* stream);

/* The same over an fp8 (e4m3fn) cache, with pa_decode_fp8's scales.        */
pa_status pa_decode_cascade_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                                int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                int32_t max_blocks_per_seq, const pa_cascade_device_plan* plan, float scale,
                                float k_scale, float v_scale, float* out, int32_t partition_tokens,
                                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_CASCADE_H_ */
