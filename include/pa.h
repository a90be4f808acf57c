/*
 * pa.h - paged-attention decode over a block-table KV cache, for AMD
 * Instinct MI355X (gfx950).  C ABI of libpa.so.
 *
 * The operation (from the pages this library follows):
 *   - The KV cache is a pool of fixed-size physical blocks of block_size
 *     tokens; each sequence has a block table mapping its logical block i to
 *     a physical block, and token i of a sequence lives at offset
 *     i % block_size of physical block table[i / block_size]
 *     (rajatmohan.com serving design, "Paging, because contiguous allocation
 *     is a disaster"; "Taming the token torrent", "The Block Table Logic").
 *   - The block tables live on the GPU as a device tensor and the kernel
 *     looks up its own block addresses ("Taming the token torrent", "The
 *     Metadata Bottleneck").
 *   - Decode runs one query token per sequence, walks the sequence's block
 *     table and performs scaled dot-product attention over the gathered
 *     blocks ("Taming the token torrent", "Custom PagedAttention Kernels").
 *     Query head i reads KV head i / (num_q_heads / num_kv_heads)
 *     ("KV Cache Engineering for LLM Serving", section 1, GQA and MQA).
 *   - Several block tables may name the same physical block when sequences
 *     share a prefix; the kernels only read blocks, so sharing needs nothing
 *     from them (same page, section 11; "Taming the token torrent",
 *     "Implementing Radix Tree Prefix Caching").
 *   - An fp8 cache stores each value as an OCP e4m3fn code with one fp32
 *     scale per tensor ("KV Cache Engineering for LLM Serving", section 8,
 *     Quantization; rajatmohan.com, "Offloading and the memory hierarchy").
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, allocated, owned and freed by
 *     the caller.  The library never allocates or frees device memory and
 *     keeps no per-call state (the one exception is pa_decode_noalloc's
 *     static scratch array); sizes are element counts unless named _bytes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without synchronising.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is launched and a negative pa_status is returned.
 *     Device-resident data (slots, block ids, sequence lengths) is checked
 *     inside the kernels: an out-of-range slot is skipped, a sequence whose
 *     length exceeds max_blocks_per_seq * block_size or whose block table
 *     names a block outside [0, num_blocks) gets NaN output for all of its
 *     query heads; nothing is read or written outside the given buffers.
 *   - Calls on one stream may overlap nothing they share; calls on different
 *     streams that write the same cache slots or the same workspace race.
 *
 * Cache layout (both caches have num_blocks * num_kv_heads * block_size *
 * head_dim elements; block_size is a multiple of 16).  A block is split
 * into sub-blocks of 16 tokens; with X = 16 bytes / element size (X = 8 for
 * bf16, 16 for fp8) and R = X / 4 (2 for bf16, 4 for fp8):
 *     K element (block b, kv head h, token t, dim d) is at
 *         [b][h][t / 16][d / X][t % 16][d % X]
 *     V element (b, h, t, d) is at
 *         [b][h][t / 16][d / 16R][d % 16][(t % 16) / 4][(d / 16) % R][t % 4]
 * so each 16-token sub-block of one head is one contiguous tile of
 * 16 * head_dim elements for K and for V, ordered so that the decode
 * kernel reads every tile with whole 16-byte loads straight into its
 * matrix-core operands.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 4

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  PA_ERR_SHAPE = -2,       /* sizes inconsistent or out of range               */
  PA_ERR_UNSUPPORTED = -3, /* head_dim, block_size or group size not built     */
  PA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required          */
  PA_ERR_LAUNCH = -5,      /* the HIP runtime reported an error                */
  PA_ERR_DEVICE = -6,      /* no gfx950 device current, or a query failed      */
  PA_ERR_NO_BLOCKS = -7,   /* block manager: the free list is too short         */
  PA_ERR_NOT_FOUND = -8,   /* block manager: unknown (or already used) seq id   */
  PA_ERR_SWAPPED = -9,     /* block manager: the sequence is (not) swapped out  */
  PA_ERR_HOST_MEMORY = -10 /* a host buffer is not pinned (hipHostMalloc) memory */
} pa_status;

/* Geometry of one layer's KV cache.
 *   num_blocks   physical blocks in the pool (>= 1)
 *   block_size   tokens per block: 16, 32, 48, ... 256 (multiple of 16)
 *   num_kv_heads KV heads (>= 1)
 *   head_dim     64 or 128                                                  */
typedef struct pa_cache_desc {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
} pa_cache_desc;

/* Slot scatter, bf16 cache.
 * For each new token j < num_tokens with slot = slot_mapping[j]:
 *   if 0 <= slot < num_blocks * block_size, with b = slot / block_size and
 *   o = slot % block_size, copies k[j][h][:] into K at (b, h, o, :) and
 *   v[j][h][:] into V at (b, h, o, :) for every KV head h, bit for bit;
 *   a negative (or out-of-range) slot skips the token.
 * A slot is a physical token position, block * block_size + offset
 * ("Taming the token torrent", "The Block Table Logic").
 *   k, v          [num_tokens][num_kv_heads][head_dim] bf16, contiguous
 *   slot_mapping  [num_tokens] int64
 *   k_cache, v_cache  bf16 caches in the layout above, written in place
 * Two tokens with the same slot in one call: which one lands is undefined.
 * num_tokens == 0 is a no-op that returns PA_OK.                            */
pa_status pa_cache_write(const pa_cache_desc* cache, const void* k, const void* v,
                         const int64_t* slot_mapping, int32_t num_tokens,
                         void* k_cache, void* v_cache, void* stream);

/* Slot scatter into an fp8 (OCP e4m3fn) cache with one scale per tensor.
 * As pa_cache_write, except each bf16 value x is stored as the e4m3fn code
 * of y = x * inv, inv = 1.0f / scale (float32, correctly rounded, computed
 * on the host), y rounded to float32 and then to the nearest e4m3fn value
 * with ties to even, saturating at +-448; NaN is stored as 0x7F with the
 * input's sign bit.  The value a code stands for is e4m3(code) * scale
 * ("KV Cache Engineering for LLM Serving", section 8: divide by the scale,
 * round, clip to the largest code).
 *   k_scale, v_scale  finite and > 0, else PA_ERR_SHAPE                     */
pa_status pa_cache_write_fp8(const pa_cache_desc* cache, const void* k, const void* v,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             void* k_cache, void* v_cache,
                             float k_scale, float v_scale, void* stream);

/* Bytes of device workspace pa_decode / pa_decode_fp8 need for these sizes
 * on the current device (the same value for both).  Returns 0 when the
 * sizes are invalid or no gfx950 device is current.  partition_tokens: as
 * for pa_decode.                                                            */
size_t pa_decode_workspace_size(const pa_cache_desc* cache, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_blocks_per_seq,
                                int32_t partition_tokens);

/* Zero-fill a decode workspace on `stream` (a small fill kernel, so it may
 * be captured in a HIP graph).  Call once after allocating a workspace, or
 * after a call that did not run to completion.  workspace_bytes == 0 is a
 * no-op.                                                                    */
pa_status pa_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Counts, on `stream`, the non-zero merge counters of a decode workspace
 * (the first max(U, 16384) * 4 + 65,536 bytes, U = num_seqs * num_kv_heads,
 * as pa_decode describes) and stores the count in *nonzero (DEVICE int32,
 * written when the stream reaches the call).  Every call that ran to
 * completion leaves them at zero, so a non-zero count means the workspace
 * was not zero-filled or a call on it did not complete: zero-fill it again
 * (pa_decode_workspace_init) before the next decode.  For a workspace used
 * with several sizes, pass the largest U.  PA_ERR_NULL for NULL pointers,
 * PA_ERR_SHAPE for num_seqs < 0 or num_kv_heads <= 0, PA_ERR_WORKSPACE when
 * workspace_bytes is smaller than the counter region.                       */
pa_status pa_decode_workspace_check(const void* workspace, size_t workspace_bytes, int32_t num_seqs,
                                    int32_t num_kv_heads, int32_t* nonzero, void* stream);

/* Paged-attention decode, bf16 cache.
 * For every sequence s < num_seqs and query head i < num_q_heads, with
 * h = i / (num_q_heads / num_kv_heads) and L = seq_lens[s]:
 *   out[s][i][:] = sum_t w_t V_s[t][h][:],
 *   w = softmax_t(scale * dot(q[s][i][:], K_s[t][h][:])), t in [0, L),
 * where K_s[t] / V_s[t] are read from block block_tables[s][t / block_size]
 * at offset t % block_size.  L == 0 gives zeros.  seq_lens includes the
 * token written this step (write it with pa_cache_write first, or write and
 * decode in one launch with pa_decode_append).
 *   q             [num_seqs][num_q_heads][head_dim] bf16
 *   block_tables  [num_seqs][max_blocks_per_seq] int32; entries past
 *                 ceil(L / block_size) are never read
 *   seq_lens      [num_seqs] int32
 *   out           [num_seqs][num_q_heads][head_dim] float32
 *   num_q_heads % num_kv_heads == 0 and num_q_heads / num_kv_heads <= 16,
 *   else PA_ERR_SHAPE / PA_ERR_UNSUPPORTED.
 * Long sequences are split across wavefronts into partitions of
 * partition_tokens tokens (a multiple of 16; 0 = choose from the device's
 * resident-wave count so every wavefront gets an equal share), and the
 * partial softmax states are merged with a log-sum-exp reduction inside the
 * same kernel launch.
 *   workspace     device buffer of >= pa_decode_workspace_size(...) bytes,
 *                 zero-filled before its first use (pa_decode_workspace_init
 *                 or any zero fill).  Its first max(U, 16384) * 4 + 65,536
 *                 bytes, U = num_seqs * num_kv_heads, hold merge counters:
 *                 one per (sequence, KV head) unit, then 16,384 for the
 *                 groups of pieces a long unit's merge tree counts; every
 *                 call that runs to completion leaves them at zero.  The
 *                 rest holds partial results that each call writes before
 *                 reading.  So one workspace serves any number of calls of
 *                 any sizes that fit (any partition_tokens, window, dtype,
 *                 group or head_dim) as long as U <= 16384 in each: their
 *                 counters all lie in the same first 128 KiB, which nothing
 *                 else uses.  A call with U > 16384 needs a workspace
 *                 zero-filled since it was last used with a different U, and
 *                 so does any call after one that did not run to
 *                 completion.  A workspace must not be shared by calls that
 *                 may run at the same time (different streams).
 * Results differ from exact arithmetic only by float32 rounding.            */
pa_status pa_decode(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                    int32_t num_q_heads, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, float scale, float* out,
                    int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Paged-attention decode, fp8 (e4m3fn) cache with per-tensor scales.
 * As pa_decode with K_s = e4m3(code) * k_scale and V_s = e4m3(code) *
 * v_scale; codes are widened exactly on load, k_scale is folded into the
 * logit scale and v_scale into the output.  Scales finite and > 0.          */
pa_status pa_decode_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                        int32_t num_q_heads, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, float scale, float k_scale, float v_scale,
                        float* out, int32_t partition_tokens, void* workspace,
                        size_t workspace_bytes, void* stream);

/* pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same decode, with no workspace argument.  Its workspace is a scratch array
 * of 32 MiB inside the library's device code: each GPU the library's code is
 * loaded on holds its own copy until the process ends, and the call itself
 * calls no allocator.  Each call first clears the array's merge counters with a
 * fill kernel on `stream` (two launches per call).  Calls whose workspace
 * (pa_decode_workspace_size, bf16) exceeds 32 MiB return PA_ERR_WORKSPACE
 * and launch nothing: with the automatic split every shape pa_decode takes
 * fits, and fixed partitions fit up to about 30 MiB of partial records.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or different host threads) race and give
 * undefined results.  Arguments and results are pa_decode's, bit for bit
 * with the same partition_tokens.                                          */
pa_status pa_decode_noalloc(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                            int32_t num_q_heads, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* seq_lens, float scale, float* out,
                            int32_t partition_tokens, void* stream);

/* Sliding-window decode: as pa_decode / pa_decode_fp8, except that each
 * sequence attends only to its last `window` tokens, positions
 * [max(0, L - window), L); window == 0 attends to all of them (the same
 * result as pa_decode).  A local layer keeps only the most recent `window`
 * positions: each new token drops the oldest once the window is full
 * ("KV Cache Engineering for LLM Serving", section 3, sliding windows).
 * Block-table entries of blocks that hold no position of the window are
 * never read (they may be -1, e.g. after pa_bm_trim released the blocks).
 * window < 0 gives PA_ERR_SHAPE.                                            */
pa_status pa_decode_window(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                           int32_t num_q_heads, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t window, float scale, float* out,
                           int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                           void* stream);
pa_status pa_decode_window_fp8(const pa_cache_desc* cache, const void* q, int32_t num_seqs,
                               int32_t num_q_heads, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* seq_lens, int32_t window, float scale,
                               float k_scale, float v_scale, float* out, int32_t partition_tokens,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Fused append and decode: one launch that does what pa_cache_write (or
 * pa_cache_write_fp8) of each sequence's new token followed by
 * pa_decode_window (or pa_decode_window_fp8) does.  The new token of
 * sequence s is its last position, L - 1 with L = seq_lens[s] (the length
 * counts it): it is written at offset (L - 1) % block_size of block
 * block_tables[s][(L - 1) / block_size], for every KV head, and attended to
 * with the rest.  A decode step appends the token's K and V to the sequence's
 * cache and then attends over all of it ("Taming the token torrent", "The
 * Block Table Logic"; "KV Cache Engineering for LLM Serving", section 1).
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim] bf16, contiguous
 *   k_cache, v_cache  written in place (the new token's row only)
 *   window        as for pa_decode_window (0 = every token)
 *   fp8: k_scale, v_scale serve both the write (codes of x / scale, rounded
 *   as pa_cache_write_fp8 rounds them) and the read.
 * The caches and `out` are bit for bit those of the two calls it replaces
 * (same partition_tokens, same workspace size).  Sequences with L == 0 write
 * nothing and give zeros; an invalid L, or a block id outside the pool,
 * writes nothing and gives NaN rows, as for pa_decode.
 * The block that receives a sequence's new token must not appear in another
 * sequence's block table in the same call (a sequence appends into a block
 * it owns alone, as copy-on-write ensures); if it does, the outputs of the
 * sequences that share it are undefined.
 * workspace: as for pa_decode (pa_decode_workspace_size).                   */
pa_status pa_decode_append(const pa_cache_desc* cache, const void* q, const void* k_new,
                           const void* v_new, int32_t num_seqs, int32_t num_q_heads,
                           void* k_cache, void* v_cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t window,
                           float scale, float* out, int32_t partition_tokens, void* workspace,
                           size_t workspace_bytes, void* stream);
pa_status pa_decode_append_fp8(const pa_cache_desc* cache, const void* q, const void* k_new,
                               const void* v_new, int32_t num_seqs, int32_t num_q_heads,
                               void* k_cache, void* v_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens,
                               int32_t window, float scale, float k_scale, float v_scale,
                               float* out, int32_t partition_tokens, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Local-layer decode from ring tables ("KV Cache Engineering for LLM
 * Serving", section 3, sliding windows: a local layer keeps only its most
 * recent `window` positions, each new one displacing the oldest).  Each
 * sequence's table row is a ring of ring_entries block ids: logical block
 * b of the sequence (positions b * block_size ..) is
 * ring_tables[s][b % ring_entries], so the row stays ring_entries wide
 * however long the sequence grows, and the block that falls out of the
 * window is the one its next block reuses (pa_bm_add_ring_sequence keeps
 * such rows).  Otherwise as pa_decode_window / pa_decode_window_fp8: each
 * sequence attends to positions [max(0, L - window), L).
 *   ring_tables   [num_seqs][ring_entries] int32; only the entries of the
 *                 blocks holding a position of the window are read
 *   ring_entries  >= ceil(window / block_size) + 1 (every block a window
 *                 can span has its own entry), else PA_ERR_SHAPE
 *   window        >= 1, else PA_ERR_SHAPE
 *   seq_lens      any L >= 0 up to INT32_MAX - 16 (no table bound); larger
 *                 or negative L gives NaN rows
 *   k_new, v_new  both NULL: decode only, the caches are not written.  Both
 *                 non-NULL ([num_seqs][num_kv_heads][head_dim] bf16): fused
 *                 append as pa_decode_append, the new token (position L - 1)
 *                 going to offset (L - 1) % block_size of block
 *                 ring_tables[s][((L - 1) / block_size) % ring_entries].  One
 *                 NULL and one not: PA_ERR_NULL.
 *   workspace     as for pa_decode, sized by pa_decode_workspace_size with
 *                 max_blocks_per_seq = ring_entries.
 * The output is pa_decode_window's on the linear table the ring stands for,
 * bit for bit with the same partition_tokens and workspace size.            */
pa_status pa_decode_ring(const pa_cache_desc* cache, const void* q, const void* k_new,
                         const void* v_new, int32_t num_seqs, int32_t num_q_heads, void* k_cache,
                         void* v_cache, const int32_t* ring_tables, int32_t ring_entries,
                         const int32_t* seq_lens, int32_t window, float scale, float* out,
                         int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                         void* stream);
pa_status pa_decode_ring_fp8(const pa_cache_desc* cache, const void* q, const void* k_new,
                             const void* v_new, int32_t num_seqs, int32_t num_q_heads,
                             void* k_cache, void* v_cache, const int32_t* ring_tables,
                             int32_t ring_entries, const int32_t* seq_lens, int32_t window,
                             float scale, float k_scale, float v_scale, float* out,
                             int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Human-readable name of a status code (static string, never NULL).        */
const char* pa_status_string(pa_status status);

/* PA_ABI_VERSION of the built library.                                      */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
